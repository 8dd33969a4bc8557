// attn_fwd.hip -- fused attention forward for AMD Instinct MI355X (gfx950).
//
// O = softmax(Q K^T * scale [+ causal mask]) V  (the attention equation of
// page "Shape-Aware Attention", section "Inspiration") with online softmax: each query row keeps
// a running maximum m, a running sum l and an fp32 accumulator across key/value
// blocks, rescaling when the maximum grows (page "GPU Kernel for a Transformer
// Layer", section "What we learned"), so no [S_q, S_kv] score matrix exists.
// Causal masking is applied inside the kernel, only on the blocks that need it,
// and key blocks wholly above the diagonal are never loaded (same page, section
// "How we built it", for the causal kernel).  The chunked entry point enqueues
// query windows against the valid prefix of a K/V cache (page "Roofline",
// section "How we built it").
//
// Work decomposition (both element types)
//   workgroup = 4 wavefronts x 32 query rows = BM = 128 rows of one (b, h);
//   small grids split each tile's keys between two such wave groups (eight
//   wavefronts), or, where that leaves CUs unbalanced, take 64-row tiles of
//   2 query groups x 2 key halves (four wavefronts); calls with at most 32
//   query rows per head take 32-row tiles of one query group x 2 key halves;
//   per iteration a wave group stages BN = 64 keys of K and V in LDS (direct
//   global-to-LDS copies, 16 bytes per lane, into three stages -- two with
//   the key split);
//   each wave computes S^T = K Q^T on MFMA so that a lane owns ONE query row
//   (lane % 32) and 16 keys per 32-key block: the row max and row sum are
//   in-lane plus one exchange between the two half-waves (v_permlane32_swap);
//   P^T feeds the B operand of O^T = V^T P^T straight from registers; the O^T
//   accumulator is also per-lane-row, so rescaling by exp2(m_old - m_new) is a
//   per-lane multiply.
//   16-bit inputs: v_mfma_f32_32x32x16_{bf16,f16}; V^T operands come from
//   ds_read_b64_tr_b16 on the natural [key][d] LDS tile.
//   fp32 inputs: v_mfma_f32_32x32x2f32 (true fp32; gfx950 has no xf32 MFMA).
//
// Softmax numerics: scores, m, l and the accumulator are fp32.  exp(x) is
// evaluated as exp2(x * log2 e) with log2 e folded into the score scale (one
// FMA per score).  The exponent offset m of a row is any value at which the
// probabilities exp2(s - m) stay in range; in exact arithmetic it cancels
// between numerator and denominator.  It is set from the row maximum until
// every row of the wave has one, and afterwards left alone: a block's
// probabilities are taken with the current offset and only if some row's sum
// over the block exceeds 2^16 (or is not finite: an fp16 probability that
// overflowed) are the block's scores recomputed, their maximum taken and the
// offset raised to it when that maximum exceeds it by more than 2^8 (then
// acc and l are rescaled by exp2(m_old - m_new)).  Steady-state blocks
// therefore need neither the row maximum nor a rescale, and every probability
// fed to the P V product is <= 2^16 and finite in fp16.  Probabilities are
// rounded to bf16/fp16 once, as the MFMA operand of the P V product, and l
// sums those rounded values on the matrix cores: a 16x16x32 MFMA whose A
// operand is a fixed pattern of ones and whose B operand is the P operand
// itself (so the normalised weights are exactly the ones P V applies).  fp32
// inputs keep fp32 probabilities, sum them with fp32 adds and take the
// maximum on every block (their fp32 MFMAs dominate; the lazy 2^8 rule still
// skips most rescales).
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <mutex>
#include <type_traits>

#include "attn.h"
#include "gfx950.h"
#include "host_common.h"

namespace {

constexpr int HEAD_DIM = 64;
constexpr int BM = 128;        // query rows per workgroup
constexpr int BN = 64;         // keys per iteration
constexpr int MAX_SPLIT = 1024;          // key ranges per call, at most
constexpr int SPLIT_MIN_KV_TILES = 16;   // the automatic split leaves shorter key chains whole
constexpr int NTHREADS = 256;  // 4 wavefronts of 64
constexpr float LAZY_TH = 8.0f;       // log2 headroom before the offset is raised
constexpr float ROW_LIMIT = 65536.0f;  // largest 64-key row sum (16-bit paths) taken without a max

// ---------------------------------------------------------------------------
// Schedule: blockIdx.x -> (head, query rows [row0, row1)).
// Windows are enqueued heaviest first (the last window sees the longest key
// prefix when causal).  Inside a window, causal calls on short caches go
// tile-major: every head's last (heaviest) 128-row tile, then every head's
// next one, so the dispatcher approximates longest-job-first.  Otherwise
// (equal-cost tiles, or long caches) windows go head-major: one head's tiles
// back to back, last tile first, so the tiles sharing a K/V prefix run
// together while it is in L2.  When B*H is a multiple of 8, head
// h only runs on XCD h % 8 (workgroups are dealt to the 8 XCDs round-robin by
// id), so the query tiles of one head share that XCD's L2.
// ---------------------------------------------------------------------------
constexpr int TILE_MAJOR_MAX_KV = 8192;  // cache rows up to which causal windows go tile-major

struct Sched {
  int bm;          // query rows per workgroup (128, or 64 for the key split on small grids)
  int S_q;
  int chunk;       // rows per window
  int n_win;       // windows
  int tf;          // tiles per full window
  int tl;          // tiles in the last window
  int heads;       // heads enumerated per decode group
  int groups;      // 8 (XCD-grouped) or 1
  int tile_major;  // order inside a window
};

__host__ __device__ inline void decode_tile(const Sched& s, int b, int& head, int& row0, int& row1) {
  int grp = 0, L = b;
  if (s.groups == 8) {
    grp = b & 7;
    L = b >> 3;
  }
  const int last = s.n_win - 1;
  const int n_last = s.heads * s.tl;
  int w, rem, tw;  // window, position inside it, tiles per head in it
  if (L < n_last) {
    w = last;
    rem = L;
    tw = s.tl;
  } else {
    const int L2 = L - n_last;
    const int per = s.heads * s.tf;
    const int wi = L2 / per;
    rem = L2 - wi * per;
    w = last - 1 - wi;
    tw = s.tf;
  }
  int j, t;
  if (s.tile_major) {
    t = tw - 1 - rem / s.heads;
    j = rem - (rem / s.heads) * s.heads;
  } else {
    j = rem / tw;
    t = tw - 1 - (rem - j * tw);
  }
  head = j * s.groups + grp;
  const int wstart = w * s.chunk;
  const int wend = min(s.S_q, wstart + s.chunk);
  row0 = wstart + t * s.bm;
  row1 = min(wend, row0 + s.bm);
}

template <typename T>
struct Params {
  const T* q;
  const T* k;
  const T* v;
  T* o;
  int64_t q_head_stride;   // S_q * 64 elements
  int64_t kv_head_stride;  // S_kv * 64 elements
  int S_q;
  int kv_len;
  float c;          // |scale| * log2(e)
  unsigned q_flip;  // XOR mask on Q's 32-bit words: sign flip for negative scale
  Sched s;
  const int* kv_lens;  // per-sequence valid K/V rows (device, B values) or null: kv_len for all
  int H;
  int S_kv;
  // Key split across workgroups (ws_acc null: none).  Split s covers keys
  // [s * split_span, (s + 1) * split_span); its workgroups are blocks
  // s * base_grid .. +base_grid-1, and write the unnormalised partial state of
  // each row (index (s * bh + head) * S_q + row) for the merge kernel.
  float* ws_acc;   // [n_split][bh * S_q][64] fp32 acc
  float* ws_ml;    // [n_split][bh * S_q][2] fp32 (offset m, row sum l)
  int split_span;  // keys per split
  int base_grid;   // workgroups per split
  int bh;          // B * H
};

__device__ __forceinline__ float other_half(float x) {
  // value held by lane l ^ 32
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(threadIdx.x & 32 ? r[0] : r[1]);
}

__device__ __forceinline__ float max_halves(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// True if the predicate holds on some active lane: the ballot's lane mask is
// tested directly (__any converts the predicate to an integer first, two
// extra vector instructions).
__device__ __forceinline__ bool any_lane(bool p) { return __builtin_amdgcn_ballot_w64(p) != 0; }

// Online-softmax bookkeeping for one tile, shared by every element type.
// s holds the raw scores of NB 32-key blocks (16 per lane per block, -inf where
// masked).  Takes the row maximum (in-lane, then across the two half-waves),
// raises the exponent offset m only when the tile exceeds it by more than 2^8
// (then rescales acc and l by exp2(m_old - m_new) for the whole wave), and
// returns the offset to subtract: 0 while the row has seen no visible key.
// lx: the 16-bit kernels' matrix-core row-sum accumulator (register 0 is
// this lane's row), rescaled with l; null for fp32.
template <int NB>
__device__ __forceinline__ float online_offset(const f32x16 (&s)[NB], f32x16 (&acc)[2], float& m, float& l,
                                               const float cc, f32x4* lx = nullptr) {
  float mx[NB];
#pragma unroll
  for (int kb = 0; kb < NB; ++kb) {  // one chain per block, in two halves
    float a = fmaxf(s[kb][0], s[kb][1]), b = fmaxf(s[kb][8], s[kb][9]);
#pragma unroll
    for (int r = 2; r < 8; ++r) {
      a = fmaxf(a, s[kb][r]);
      b = fmaxf(b, s[kb][r + 8]);
    }
    mx[kb] = fmaxf(a, b);
  }
  float x = mx[0];
#pragma unroll
  for (int kb = 1; kb < NB; ++kb) x = fmaxf(x, mx[kb]);
  x = max_halves(x);
  const float xc = (x == -INFINITY) ? -INFINITY : x * cc;
  const bool raise = xc > m + LAZY_TH;
  if (any_lane(raise)) {
    // Raising lanes scale by exp2(m - xc) (0 when m was -inf); the others keep
    // their offset and scale by exactly 1 (m may still be -inf there: rows
    // that have not seen a visible key yet, so m - m would be NaN).
    const float m_new = raise ? xc : m;
    const float alpha = raise ? fast_exp2(m - xc) : 1.f;
    l *= alpha;
    if (lx) (*lx)[0] *= alpha;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      acc[0][r] *= alpha;
      acc[1][r] *= alpha;
    }
    m = m_new;
  }
  return (m == -INFINITY) ? 0.f : m;
}

// ---------------------------------------------------------------------------
// 16-bit element types
// ---------------------------------------------------------------------------
// V is read with ds_read_b64_tr_b16: per 16-lane group, 4 consecutive rows x
// 2 adjacent chunks; shifting the chunk pair by 2*(row & 3) spreads them over 8
// distinct chunks.
__device__ __forceinline__ int v16_off(int row, int c16) {
  return row * 128 + ((c16 ^ ((row & 3) << 1)) << 4);
}

// Probabilities of one tile for the 16-bit path: P = exp2(s*c - moff) in fp32,
// RNE-packed to 16 bits in the B-operand layout of the P V product (pw[kb][u]
// word q holds keys 8u + 2q, 8u + 2q + 1 of block kb, k-slots 8hf + 2q, +1).
template <typename T, int NB>
__device__ __forceinline__ void probs16(const f32x16 (&s)[NB], const float cc, const float moff,
                                        u32x4 (&pw)[NB][2]) {
  typedef Half16<T> H;
#pragma unroll
  for (int kb = 0; kb < NB; ++kb)
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int r = 8 * u + 2 * q;
        const float e0 = fast_exp2(__builtin_fmaf(s[kb][r], cc, -moff));
        const float e1 = fast_exp2(__builtin_fmaf(s[kb][r + 1], cc, -moff));
        pw[kb][u][q] = H::pack2(e0, e1);
      }
}

// Row sums of the packed probabilities on the matrix cores.  Step (kb, u) of
// pw is 64 lanes x 8 values, lane (c, hf) holding 8 of query c's; as the B
// operand of a 16x16x32 MFMA (B[k][j] at lane j + 16(k/8), element k%8) it is
// column j = lane % 16 with k-groups from lanes j, j+16, j+32, j+48, i.e.
// queries j, j+16, j, j+16.  `ones` (A[i][k] at lane i + 16(k/8)) is 1 in
// rows 0 and 8 for k-groups 0 and 2 and in rows 4 and 12 for k-groups 1 and
// 3, 0 elsewhere, so C[0][j] and C[8][j] are query j's sum and C[4][j],
// C[12][j] query j+16's; with C[i][j] at lane j + 16(i/4), register i%4,
// register 0 of every lane holds its own query's sum over the step's 16 keys
// (both half-waves' keys).  Returns rs plus the tile's row sums (register 0).
template <typename T, int NB>
__device__ __forceinline__ f32x4 rowsum16_acc(const u32x4 (&pw)[NB][2], const typename Half16<T>::vec8& ones,
                                              f32x4 rs) {
  typedef Half16<T> H;
#pragma unroll
  for (int kb = 0; kb < NB; ++kb)
#pragma unroll
    for (int u = 0; u < 2; ++u) rs = H::mfma16(ones, __builtin_bit_cast(typename H::vec8, pw[kb][u]), rs);
  return rs;
}


// The A operand of rowsum16 for this lane: ones where (lane % 16) % 8 is 4 *
// ((lane / 16) % 2) and lane % 4 is 0 (lanes 0, 8, 20, 28, 32, 40, 52, 60).
template <typename T>
__device__ __forceinline__ typename Half16<T>::vec8 rowsum_ones(const int lane) {
  const unsigned w = ((lane & 7) == 4 * ((lane >> 4) & 1) && (lane & 3) == 0) ? Half16<T>::ONE2 : 0u;
  const u32x4 x = {w, w, w, w};
  return __builtin_bit_cast(typename Half16<T>::vec8, x);
}

// The softmax half of one wave's work on one 64-key tile: S^T = K Q^T on
// MFMA, the online-softmax update and the packed probabilities pw (the B
// operands of the tile's P V product, pv16).  TWO: the tile's second 32-key
// block is visible to some row of this wave (false only on causal diagonal
// tiles and at the cache end).  MASK: some key of the tile is invisible to
// some row.  SPEC: take the probabilities at the current offset first (false
// for a wave's first tile, whose offsets are not set yet: straight to the
// maximum).  MSET: every lane's offset is known to be set (after a first tile
// that every row of the wave sees in full), so only the block sums are
// checked.
// lx: the row sum (register 0), accumulated on the matrix cores; a tile reads
// its own sum as the increase of lx.  online_offset rescales lx with acc; l is
// unused (fp32 keeps its sums there).
template <typename T, bool TWO, bool MASK, bool CAUSAL, bool SPEC = true, bool MSET = false>
__device__ __forceinline__ void softmax16(const char* ks, const typename Half16<T>::vec8 (&qop)[4],
                                          const typename Half16<T>::vec8& ones, f32x16 (&acc)[2], float& m,
                                          float& l, f32x4& lx, const float cc, const int kv0, const int kv_len,
                                          const int pos, const int lane, u32x4 (&pw)[TWO ? 2 : 1][2]) {
  typedef Half16<T> H;
  typedef typename H::vec8 vec8;
  constexpr int NB = TWO ? 2 : 1;
  const int c = lane & 31, hf = lane >> 5;

  // S^T = K Q^T; k-step t: lane holds K[32kb + c][32hf + 8t .. +7].  Keys
  // this lane's row cannot see get -inf (exp2(-inf) = 0); only diagonal and
  // cache-end tiles carry the mask.
  auto scores = [&](f32x16 (&s)[NB], const int k0) {
#pragma unroll
    for (int kb = 0; kb < NB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) s[kb][r] = 0.f;
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int kb = 0; kb < NB; ++kb) {
        const vec8 a = *reinterpret_cast<const vec8*>(ks + k16_off(32 * kb + c, 4 * hf + t));
        s[kb] = H::mfma(a, qop[t], s[kb]);
      }
    if constexpr (MASK) {
#pragma unroll
      for (int kb = 0; kb < NB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = k0 + 32 * kb + 8 * (r >> 2) + 4 * hf + (r & 3);
          const bool vis = key < kv_len && (!CAUSAL || key <= pos);
          s[kb][r] = vis ? s[kb][r] : -INFINITY;
        }
    }
  };
  f32x16 s[NB];
  scores(s, kv0);

  // Take the probabilities at the current offset.  If some lane's offset is
  // not set yet (m = -inf: its row has seen no key) or its row's block sum is
  // out of range (above 2^16, or not finite), redo the tile through the
  // maximum: re-read K (s is consumed by then, so no score register lives
  // across the branch), raise the offset, recompute.  The test is per lane
  // and comes after the probabilities, so the steady case is one
  // straight-line block; one call site keeps a single rescale point for acc.
  if constexpr (SPEC) {
    probs16<T, NB>(s, cc, m, pw);
    f32x4 lnew = rowsum16_acc<T, NB>(pw, ones, lx);
    const float ts = lnew[0] - lx[0];  // this tile's row sum (>= 0, or inf / NaN)
    // Out of range: above 2^16, infinite, or NaN.  A NaN appears when an fp16
    // probability overflowed (inf) and meets a zero of the ones pattern in
    // another row's sum, so every lane of that pair may hold NaN; the sums are
    // never negative, so comparing the bit patterns as unsigned integers
    // catches +inf and NaN of either sign whatever the compiler assumes about
    // NaN (the device code is built with -fno-honor-nans).  lx grows by at
    // most 2^16 per tile, so the increase is exact to far better than the
    // limit.
    const bool out_of_range = __float_as_uint(ts) > __float_as_uint(ROW_LIMIT);
    if (any_lane(out_of_range || (!MSET && m == -INFINITY))) {
      asm volatile("" ::: "memory");
      // An opaque copy of kv0: the masks are recomputed here rather than the
      // first pass's 32 lane masks being kept in scalar registers meanwhile.
      int k0 = kv0;
      asm volatile("" : "+v"(k0));
      f32x16 s2[NB];
      scores(s2, k0);
      const float moff = online_offset<NB>(s2, acc, m, l, cc, &lx);  // may rescale acc and lx
      probs16<T, NB>(s2, cc, moff, pw);
      lnew = rowsum16_acc<T, NB>(pw, ones, lx);
    }
    lx = lnew;
  } else {
    const float moff = online_offset<NB>(s, acc, m, l, cc, &lx);  // may rescale acc and lx
    probs16<T, NB>(s, cc, moff, pw);
    lx = rowsum16_acc<T, NB>(pw, ones, lx);
  }
}

// The P V half: O^T += V^T P^T for the tile whose probabilities are pw.  V^T
// operands are read transposed from the [key][d] tile: operand (kb, u, dt),
// k-slot 8hf + e, holds V[32kb + 16u + 8(e/4) + 4hf + e%4][32dt + c]: source
// lane s of each 16-lane group reads row kbase + s/4, columns d0 + 4(s%4)
// .. +3.  Step (kb, u) contracts keys 32kb + 16u .. +15.
template <typename T, bool TWO>
__device__ __forceinline__ void pv16(const char* vs, const u32x4 (&pw)[TWO ? 2 : 1][2], f32x16 (&acc)[2],
                                     const int lane) {
  typedef Half16<T> H;
  typedef typename H::vec8 vec8;
  constexpr int NB = TWO ? 2 : 1;
  const int g = lane >> 4, sl = lane & 15;
#pragma unroll
  for (int kb = 0; kb < NB; ++kb)
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      vec8 va[2];
#pragma unroll
      for (int dt = 0; dt < 2; ++dt) {
        const int d0 = 32 * dt + 16 * (g & 1) + 4 * (sl & 3);
        const int c16 = d0 >> 3, half = (d0 >> 2) & 1;
        const int row = 32 * kb + 16 * u + 4 * (g >> 1) + (sl >> 2);
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(i16x4, vs + v16_off(row, c16) + 8 * half));
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(i16x4, vs + v16_off(row + 8, c16) + 8 * half));
        const u32x2 lo2 = __builtin_bit_cast(u32x2, lo), hi2 = __builtin_bit_cast(u32x2, hi);
        const u32x4 aw = {lo2[0], lo2[1], hi2[0], hi2[1]};
        va[dt] = __builtin_bit_cast(vec8, aw);
      }
      const vec8 b = __builtin_bit_cast(vec8, pw[kb][u]);
#pragma unroll
      for (int dt = 0; dt < 2; ++dt) acc[dt] = H::mfma(va[dt], b, acc[dt]);
    }
}

// One wave's whole work on one 64-key tile: softmax16, then pv16 (the V^T
// operands are read after the softmax: not live during it, the 16-bit kernel
// fits three workgroups per CU at 168 VGPRs).
template <typename T, bool TWO, bool MASK, bool CAUSAL, bool SPEC = true, bool MSET = false>
__device__ __forceinline__ void tile16(const char* ks, const char* vs, const typename Half16<T>::vec8 (&qop)[4],
                                       const typename Half16<T>::vec8& ones, f32x16 (&acc)[2], float& m, float& l,
                                       f32x4& lx, const float cc, const int kv0, const int kv_len, const int pos,
                                       const int lane) {
  u32x4 pw[TWO ? 2 : 1][2];
  softmax16<T, TWO, MASK, CAUSAL, SPEC, MSET>(ks, qop, ones, acc, m, l, lx, cc, kv0, kv_len, pos, lane, pw);
  pv16<T, TWO>(vs, pw, acc, lane);
}

// ---------------------------------------------------------------------------
// fp32
// ---------------------------------------------------------------------------
// LDS tile of 64 rows x 256 bytes (64 floats) = 16 KB, 16 chunks per row.
// K is XOR-swizzled by row: the S^T operand reads take 16 consecutive rows at
// one chunk position per access.
__device__ __forceinline__ int k32_off(int row, int c16) {
  return row * 256 + ((c16 ^ (row & 15)) << 4);
}
// V is stored unswizzled: the P V operand reads take one 256-byte row per
// 32 lanes (lanes 0-31 row R, lanes 32-63 row R + 4), which is conflict-free
// as is, and fixed row offsets become immediate address offsets.

// fp32 probabilities of one tile, in place: s <- exp2(s*c - moff).  Returns
// this lane's sum of them.
template <int NB>
__device__ __forceinline__ float probs32(f32x16 (&s)[NB], const float cc, const float moff) {
  float ls[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kb = 0; kb < NB; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float e = fast_exp2(__builtin_fmaf(s[kb][r], cc, -moff));
      ls[r & 3] += e;
      s[kb][r] = e;
    }
  return (ls[0] + ls[1]) + (ls[2] + ls[3]);
}

// One wave's work on one 64-key fp32 tile (see tile16 for TWO and MASK).
// The two O^T accumulators hold interleaved columns: acc[dt] row i is
// d = 2i + dt, so one 8-byte read V[key][2c .. 2c+1] feeds both P V MFMAs.
template <bool TWO, bool MASK, bool CAUSAL>
__device__ __forceinline__ void tile32(const char* ks, const char* vs, const float (&qv)[32], f32x16 (&acc)[2],
                                       float& m, float& l, const float cc, const int kv0, const int kv_len,
                                       const int pos, const int lane) {
  constexpr int NB = TWO ? 2 : 1;
  const int c = lane & 31, hf = lane >> 5;

  // S^T = K Q^T: k-step t contracts d = 32hf + t; lane reads K[32kb + c][32hf .. +31]
  // as eight 16-byte chunks, each feeding four MFMAs.  Masked keys get -inf.
  auto scores = [&](f32x16 (&s)[NB]) {
#pragma unroll
    for (int kb = 0; kb < NB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) s[kb][r] = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      u32x4 ka[NB];
#pragma unroll
      for (int kb = 0; kb < NB; ++kb) ka[kb] = *reinterpret_cast<const u32x4*>(ks + k32_off(32 * kb + c, 8 * hf + j));
#pragma unroll
      for (int e = 0; e < 4; ++e)
#pragma unroll
        for (int kb = 0; kb < NB; ++kb)
          s[kb] = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(ka[kb][e]), qv[4 * j + e], s[kb], 0, 0, 0);
    }
    if constexpr (MASK) {
#pragma unroll
      for (int kb = 0; kb < NB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kv0 + 32 * kb + 8 * (r >> 2) + 4 * hf + (r & 3);
          const bool vis = key < kv_len && (!CAUSAL || key <= pos);
          s[kb][r] = vis ? s[kb][r] : -INFINITY;
        }
    }
  };
  f32x16 s[NB];
  scores(s);

  // V operands of block 0, read ahead of the softmax: step r of block kb
  // contracts keys 32kb + 8(r/4) + 4hf + r%4 (k-slot hf), lane (c, hf) needs
  // V[that key][2c], V[that key][2c + 1].
  const char* vlane = vs + (4 * hf) * 256 + 8 * c;
  f32x2 va[NB][16];
#pragma unroll
  for (int r = 0; r < 16; ++r)
    va[0][r] = *reinterpret_cast<const f32x2*>(vlane + (8 * (r >> 2) + (r & 3)) * 256);

  // fp32 tiles are bound by the fp32 MFMA rate: the row maximum costs less
  // than the register traffic of the max-free path, so every tile takes it.
  const float moff = online_offset<NB>(s, acc, m, l, cc);  // may rescale acc and l
  l += probs32<NB>(s, cc, moff);

  // O^T += V^T P^T, one key pair per MFMA: k-slot hf of step r is this lane's
  // probability s[kb][r].  Block 1's operands are read during block 0's MFMAs.
  if constexpr (TWO) {
#pragma unroll
    for (int r = 0; r < 16; ++r)
      va[1][r] = *reinterpret_cast<const f32x2*>(vlane + (32 + 8 * (r >> 2) + (r & 3)) * 256);
  }
#pragma unroll
  for (int kb = 0; kb < NB; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      acc[0] = __builtin_amdgcn_mfma_f32_32x32x2f32(va[kb][r][0], s[kb][r], acc[0], 0, 0, 0);
      acc[1] = __builtin_amdgcn_mfma_f32_32x32x2f32(va[kb][r][1], s[kb][r], acc[1], 0, 0, 0);
    }
}

// ---------------------------------------------------------------------------
// The kernel (all element types)
// ---------------------------------------------------------------------------
// KS = 1: 4 wavefronts, one per 32 query rows; each wave walks every key tile.
// KS = 2: 8 wavefronts; waves 4..7 take the same query rows as waves 0..3 but
// the odd 64-key tiles while waves 0..3 take the even ones, and the two
// partial (m, l, acc) states are merged through LDS at the end.  This halves
// the sequential key chain per wave when there are too few workgroups to
// fill the GPU.
//
// Pipeline: a stage holds KS consecutive 64-key tiles of K, then of V.  With
// three stages two stages are in flight while one is computed; with two, one.
// The 16-bit one-group kernel's full-tile loop runs each tile's P V one step
// late, beside the next tile's probabilities: there the previous tile stays
// resident and one stage is in flight.
//
// VARLEN: each sequence has its own key length, read from p.kv_lens (key
// padding); a row that then sees no key gets zeros.
// SPLIT: the workgroup covers one key range of its query rows (the cache is
// viewed from the range's first row on, with the causal shift of the whole
// cache) and writes the partial (m, l, acc) instead of O.
// Occupancy: three four-wave 16-bit workgroups per CU (48 KB of LDS and at
// most 168 VGPRs each), else one or two.
template <typename T, bool CAUSAL, int KS, bool VARLEN, bool SPLIT, int QG = 4>
__global__ void __launch_bounds__(64 * QG * KS, (sizeof(T) == 2 && KS == 1) ? 3 : (QG <= 2 && sizeof(T) == 2 ? 2 : 1))
    attn_fwd_kernel(Params<T> p) {
  // QG: 32-row query groups per workgroup (4: 128 rows; 2: 64 rows; 1: 32
  // rows, for at most 32 query rows per head: decode steps), the smaller
  // tiles with the key split only (2 QG waves, two workgroups per CU for
  // 16-bit types, one for fp32).
  static_assert(QG == 4 || ((QG == 2 || QG == 1) && KS == 2), "64- and 32-row tiles: key split only");
  constexpr bool F32 = sizeof(T) == 4;
  constexpr int ROWB = F32 ? 256 : 128;  // bytes per K/V row (64 elements)
  constexpr int TILE = 64 * ROWB;        // one 64-row tile of K or V
  constexpr int STAGE = 2 * KS * TILE;   // KS K tiles, then KS V tiles
  constexpr int NS = KS == 1 ? 3 : 2;    // LDS stages
  constexpr int LPR = ROWB / 16;         // lanes per row in one 16-byte-per-lane copy
  constexpr int RPC = 64 / LPR;          // rows per copy instruction
  constexpr int NCP = 64 / (QG * RPC);   // copies per wave per matrix per stage
  // Distinct arrays: reading one stage never waits for copies into another.
  __shared__ __attribute__((aligned(16))) char st0[STAGE];
  __shared__ __attribute__((aligned(16))) char st1[STAGE];
  __shared__ __attribute__((aligned(16))) char st2[NS == 3 ? STAGE : 16];

  int head, row0, row1;
  int split = 0, tile_id = blockIdx.x;
  if constexpr (SPLIT) {
    split = tile_id / p.base_grid;
    tile_id -= split * p.base_grid;
  }
  decode_tile(p.s, tile_id, head, row0, row1);

  const int tid = threadIdx.x;
  // 0 .. 4*KS-1.  Deliberately not made compiler-uniform (readfirstlane):
  // with scalar branches the per-tile variants below join in ways that make
  // the register allocator copy the accumulators in and out on every tile;
  // as exec-masked branches they stay in place.
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int qg = wave % QG;   // query group: rows 32*qg .. +31 of the tile
  const int kh = wave / QG;   // key half (KS = 2)
  const int c = lane & 31;    // query column of the S^T / O^T tiles
  const int hf = lane >> 5;   // half-wave

  const T* qh = p.q + (int64_t)head * p.q_head_stride;
  const int k_start = SPLIT ? split * p.split_span : 0;  // first key of this workgroup's range
  const T* kh_ptr = p.k + (int64_t)head * p.kv_head_stride + (int64_t)k_start * HEAD_DIM;
  const T* vh_ptr = p.v + (int64_t)head * p.kv_head_stride + (int64_t)k_start * HEAD_DIM;
  T* oh = p.o + (int64_t)head * p.q_head_stride;

  // Valid K/V rows of this head's sequence: kv_len, or its own length
  // clamped into the cache (a row that sees no key gets zeros).
  const int kv_full = VARLEN ? min(max(p.kv_lens[head / p.H], 0), p.S_kv) : p.kv_len;
  // From here on keys are counted from k_start: the range holds kv_len of
  // them, and query row r sits at position r + shift.
  const int kv_len = SPLIT ? max(0, min(kv_full, k_start + p.split_span) - k_start) : kv_full;
  const int shift = kv_full - p.S_q - k_start;
  const int kv_end0 = CAUSAL ? min(kv_len, row1 + shift) : kv_len;
  const int kv_end = (VARLEN || SPLIT) ? max(0, kv_end0) : kv_end0;
  const int n_tiles = (kv_end + BN - 1) / BN;
  const int n_super = (n_tiles + KS - 1) / KS;

  // This wave's query rows and their positions.
  const int wrow0 = row0 + qg * 32;
  const int qrow = wrow0 + c;
  const bool wave_live = wrow0 < row1;
  const int wlast = min(wrow0 + 31, row1 - 1);  // last valid row of the wave
  const int pos = qrow + shift;
  const int pos_first = wrow0 + shift;
  const int pos_last = wlast + shift;

  // Q operand (B operand of S^T = K Q^T), resident for the whole key loop.
  // 16-bit: k-step t holds Q[qrow][32hf + 8t .. +7]; fp32: k-step t holds Q[qrow][32hf + t].
  typename std::conditional<F32, float[32], typename Half16<typename std::conditional<F32, __bf16, T>::type>::vec8[4]>::type qop;

  // Tile copies: the waves of key half kh copy its 64-row tile of K and of V;
  // copy i of wave (kh, qg) fills stage rows 64 kh + RPC*(QG i + qg) .. +RPC-1,
  // lane l lands in row + l/LPR, physical chunk l%LPR and fetches the logical
  // chunk the row's swizzle maps there.  The swizzle depends only on the row
  // modulo 16, so copies of a wave whose rows differ by a multiple of 16 lie
  // as far apart in the source as in the stage (paired in issue_full).  The
  // source is a per-lane address fixed for the whole loop, advanced by the
  // super-tile's (scalar) offset; only a super-tile that crosses the cache
  // end computes clamped rows (rows past kv_len - 1 re-read row kv_len - 1:
  // finite data, and those keys are masked).
  // Stage row of copy i of the wave of thread t, and the byte offsets of the
  // lane's 16-byte chunk in a K row and a V row (swizzled).  The clamped
  // copies recompute these from an opaque copy of the thread index, so none
  // of them stays live across the key loop.
  auto copy_geom = [&](const int i, const int t, int& row, uint32_t& kc, uint32_t& vc) __attribute__((always_inline)) {
    const int ln = t & 63, wv = t >> 6;
    row = 64 * (wv / QG) + RPC * (QG * i + (wv % QG)) + ln / LPR;
    const int ph = ln % LPR;
    if constexpr (F32) {
      kc = 16 * (ph ^ (row & 15));
      vc = 16 * ph;
    } else {
      kc = 16 * (ph ^ ((row & 7) ^ ((row >> 3) & 1)));
      vc = 16 * (ph ^ ((row & 3) << 1));
    }
  };
  uint32_t kof[NCP], vof[NCP];
#pragma unroll
  for (int i = 0; i < NCP; ++i) {
    int row;
    uint32_t kc, vc;
    copy_geom(i, tid, row, kc, vc);
    kof[i] = (uint32_t)row * ROWB + kc;
    vof[i] = (uint32_t)row * ROWB + vc;
  }
  const uint32_t wdst = __builtin_amdgcn_readfirstlane((uint32_t)((64 * kh + RPC * qg) * ROWB));
  const char* kbase = reinterpret_cast<const char*>(kh_ptr);
  const char* vbase = reinterpret_cast<const char*>(vh_ptr);
  const char* kl[NCP];
  const char* vl[NCP];
#pragma unroll
  for (int i = 0; i < NCP; ++i) {
    kl[i] = kbase + kof[i];
    vl[i] = vbase + vof[i];
  }
  // A super-tile entirely below the cache end.
  // Copy i + 1 lies QG RPC rows = CSTEP bytes after copy i in the stage.
  // Copies PG apart, whose rows differ by a multiple of the swizzle period
  // (16 rows), also lie PG CSTEP bytes apart in the source: they go in pairs
  // (dma16_pair, offsets -PG CSTEP/2 and +PG CSTEP/2 around one address).
  // PG = 1 except for fp32 with 64-row tiles (copies 8 rows apart: pairs
  // (i, i + 2)).
  constexpr int CSTEP = RPC * QG * ROWB;
  constexpr int PG = (QG * RPC) % 16 == 0 ? 1 : 16 / (QG * RPC);
  constexpr int PSTEP = PG * CSTEP;
  static_assert((PSTEP == 4096 || PSTEP == 2048) && NCP % (2 * PG) == 0, "paired tile copies");
  auto issue_full = [&](char* st, int super) __attribute__((always_inline)) {
    const uint32_t mk = lds_addr(st) + wdst, mv = mk + KS * TILE;
    const int64_t off = (int64_t)super * KS * BN * ROWB;
#pragma unroll
    for (int i = 0; i < NCP; ++i) {
      if ((i / PG) % 2 != 0) continue;  // the second copy of a pair
      dma16_pair<PSTEP / 2>(kl[i] + (off + PSTEP / 2), mk + i * CSTEP + PSTEP / 2);
      dma16_pair<PSTEP / 2>(vl[i] + (off + PSTEP / 2), mv + i * CSTEP + PSTEP / 2);
    }
  };
  auto issue = [&](char* st, int super) __attribute__((always_inline)) {
    const int kv0 = super * KS * BN;
    if (kv0 + KS * BN <= kv_len) {
      issue_full(st, super);
    } else {
      const uint32_t mk = lds_addr(st) + wdst, mv = mk + KS * TILE;
      int tx = threadIdx.x;
      asm volatile("" : "+v"(tx));
#pragma unroll
      for (int i = 0; i < NCP; ++i) {
        int row;
        uint32_t kc, vc;
        copy_geom(i, tx, row, kc, vc);
        const uint32_t rb = (uint32_t)min(kv0 + row, kv_len - 1) * ROWB;
        dma16(kbase + (rb + kc), mk + i * CSTEP);
        dma16(vbase + (rb + vc), mv + i * CSTEP);
      }
    }
  };

  // Each wave copies its own 32 Q rows (whole rows, K's swizzle) into its own
  // slab of the stage that the first step refills, ahead of the first K/V
  // copies, and reads them into the MFMA operand after its first wait --
  // its own copies only, so no barrier is needed before the read -- and
  // before that step's barrier.  Whole-row copies instead of per-lane loads
  // that touch 32 rows each, and the first step waits only for what it needs.
  // Rows past the tile's end re-read its last row (never stored).
  constexpr int SLAB = 32 * ROWB;  // one wave's Q rows; the QG KS slabs fit in a stage
  static_assert(QG * KS * SLAB <= STAGE, "Q slabs");
  char* const qst = NS == 3 ? st2 : st1;
  const uint32_t wslab = __builtin_amdgcn_readfirstlane((uint32_t)(wave * SLAB));
  {
    const uint32_t mq = lds_addr(qst) + wslab;
    const char* qb = reinterpret_cast<const char*>(qh);
#pragma unroll
    for (int i = 0; i < SLAB / 1024; ++i) {
      const int row = RPC * i + lane / LPR;  // row of the slab
      const int ph = lane % LPR;
      const uint32_t cb = F32 ? 16 * (ph ^ (row & 15)) : 16 * (ph ^ ((row & 7) ^ ((row >> 3) & 1)));
      dma16(qb + ((int64_t)min(wrow0 + row, row1 - 1) * ROWB + cb), mq + i * 1024);
    }
  }
  auto read_q = [&]() __attribute__((always_inline)) {
    const char* qs = qst + wslab;
    if constexpr (F32) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        u32x4 x = *reinterpret_cast<const u32x4*>(qs + k32_off(c, 8 * hf + j));
        x ^= p.q_flip;
#pragma unroll
        for (int e = 0; e < 4; ++e) qop[4 * j + e] = __uint_as_float(x[e]);
      }
    } else {
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        u32x4 x = *reinterpret_cast<const u32x4*>(qs + k16_off(c, 4 * hf + t));
        x ^= p.q_flip;
        qop[t] = __builtin_bit_cast(typename std::remove_reference<decltype(qop[0])>::type, x);
      }
    }
  };

  f32x16 acc[2];
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    acc[0][r] = 0.f;
    acc[1][r] = 0.f;
  }
  float m = -INFINITY;  // exponent offset (log2 units), per row
  float l = 0.f;        // row sum: 16-bit, the whole row's; fp32, this lane's share
  f32x4 lx = {0.f, 0.f, 0.f, 0.f};  // 16-bit: row sums of optimistic tiles (register 0)
  // A operand of the 16-bit row sums (rowsum16).
  const auto ones = rowsum_ones<typename std::conditional<F32, __bf16, T>::type>(lane);
  const float cc = p.c;

  auto compute = [&](const char* st, int super) __attribute__((always_inline)) {
    const int t = super * KS + kh;
    if (t >= n_tiles) return;
    const int kv0 = t * BN;
    // Which 32-key blocks can some row of this wave see, and does any key of
    // the tile need masking (cache end, or past the first row's position)?
    const bool blk0 = wave_live && (!CAUSAL || kv0 <= pos_last);
    if (!blk0) return;
    const bool blk1 = kv0 + 32 < kv_len && (!CAUSAL || kv0 + 32 <= pos_last);
    const int last_key = kv0 + (blk1 ? 63 : 31);
    const bool need_mask = last_key >= kv_len || (CAUSAL && last_key > pos_first);
    const char* ks = st + kh * TILE;
    const char* vs = st + KS * TILE + kh * TILE;
    if constexpr (F32) {
      if (blk1) {
        if (need_mask)
          tile32<true, true, CAUSAL>(ks, vs, qop, acc, m, l, cc, kv0, kv_len, pos, lane);
        else
          tile32<true, false, CAUSAL>(ks, vs, qop, acc, m, l, cc, kv0, kv_len, pos, lane);
      } else {
        if (need_mask)
          tile32<false, true, CAUSAL>(ks, vs, qop, acc, m, l, cc, kv0, kv_len, pos, lane);
        else
          tile32<false, false, CAUSAL>(ks, vs, qop, acc, m, l, cc, kv0, kv_len, pos, lane);
      }
    } else {
      if (blk1) {
        if (need_mask)
          tile16<T, true, true, CAUSAL>(ks, vs, qop, ones, acc, m, l, lx, cc, kv0, kv_len, pos, lane);
        else
          tile16<T, true, false, CAUSAL>(ks, vs, qop, ones, acc, m, l, lx, cc, kv0, kv_len, pos, lane);
      } else {
        if (need_mask)
          tile16<T, false, true, CAUSAL>(ks, vs, qop, ones, acc, m, l, lx, cc, kv0, kv_len, pos, lane);
        else
          tile16<T, false, false, CAUSAL>(ks, vs, qop, ones, acc, m, l, lx, cc, kv0, kv_len, pos, lane);
      }
    }
  };

  // Tiles every wave of the workgroup sees in full (all keys below the cache
  // end and, when causal, at or before the workgroup's first row): the
  // leading super-steps made only of such tiles, whose prefetched super-tile
  // also lies entirely below the cache end, run a loop without conditions:
  // no visibility, mask or clamp logic, fixed waits, and every wave computes
  // (one whose rows all lie past the window's end is never stored).  The
  // first such tile is taken with the row maximum and gives every lane an
  // offset, so the later ones check only their block sums.
  int t_full = kv_len / BN;
  if (CAUSAL) t_full = min(t_full, (row0 + shift + 1) / BN);
  int j_full = min(t_full / KS, min(kv_len / (KS * BN), n_super) - (NS - 1));
  j_full = j_full > 0 ? j_full - j_full % NS : 0;
  auto compute_full = [&](const char* st, int super, auto spec) __attribute__((always_inline)) {
    const char* ks = st + kh * TILE;
    const char* vs = st + KS * TILE + kh * TILE;
    const int kv0 = (super * KS + kh) * BN;
    if constexpr (F32)
      tile32<true, false, CAUSAL>(ks, vs, qop, acc, m, l, cc, kv0, kv_len, pos, lane);
    else
      tile16<T, true, false, CAUSAL, decltype(spec)::value, decltype(spec)::value>(ks, vs, qop, ones, acc, m, l, lx,
                                                                                  cc, kv0, kv_len, pos, lane);
  };
  const std::true_type spec;    // offsets set (every lane): speculate
  const std::false_type first;  // a wave's first tile

  if (n_super > 0) issue(st0, 0);
  if (NS == 3 && n_super > 1) issue(st1, 1);
  // The Q rows and super-tile 0 (copied before super-tile 1).
  if constexpr (NS == 3) {
    if (n_super > 1)
      wait_vmem<2 * NCP>();
    else
      wait_vmem<0>();
  } else {
    wait_vmem<0>();
  }
  read_q();

  int j = 0;
  if constexpr (NS == 3) {
    // Stage j % 3 holds super-tile j.  At step j super-tiles j and j+1 may be
    // in flight: wait for j, barrier (everyone is done with j-1), start j+2
    // into j-1's stage, compute j.
    auto sync = [&](char* nxt, int j) __attribute__((always_inline)) {
      if (j + 1 < n_super)
        wait_vmem<2 * NCP>();
      else
        wait_vmem<0>();
      barrier_keep_dma();
      if (j + 2 < n_super) issue(nxt, j + 2);
    };
    if constexpr (!F32) {
      // 16-bit full tiles with the P V product one step behind: step j takes
      // tile j - 1's P V and then tile j's softmax, so the matrix cores have
      // independent work (the P V MFMAs) while the probabilities of tile j
      // are computed.  Tile j - 1 must stay in its stage during step j, so
      // copies run one tile ahead: step j starts tile j + 1 into the stage of
      // tile j - 2 (free once every wave has passed this step's barrier).
      u32x4 pw_prev[2][2];
      auto step = [&](char* cur, char* prev, char* nxt, int j) __attribute__((always_inline)) {
        wait_vmem<0>();
        barrier_keep_dma();
        issue_full(nxt, j + 1);
        // The P V MFMAs come first in the source so that they share the
        // basic block of this tile's probabilities (the fallback test ends
        // it); the scheduler spreads them over the probability arithmetic.
        pv16<T, true>(prev + TILE, pw_prev, acc, lane);
        u32x4 pw[2][2];
        softmax16<T, true, false, CAUSAL, true, true>(cur, qop, ones, acc, m, l, lx, cc, j * BN, kv_len, pos, lane,
                                                       pw);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int u = 0; u < 2; ++u) pw_prev[kb][u] = pw[kb][u];
      };
      if (j_full > 0) {
        // Step 0: tiles 0 and 1 are in flight; the first tile sets the offsets.
        wait_vmem<2 * NCP>();
        barrier_keep_dma();
        softmax16<T, true, false, CAUSAL, false, false>(st0, qop, ones, acc, m, l, lx, cc, 0, kv_len, pos, lane,
                                                         pw_prev);
        for (j = 1; j < j_full; j += 3) {
          step(st1, st0, st2, j);
          if (j + 1 >= j_full) {
            j += 1;
            break;
          }
          step(st2, st1, st0, j + 1);
          if (j + 2 >= j_full) {
            j += 2;
            break;
          }
          step(st0, st2, st1, j + 2);
        }
        // j == j_full, a multiple of 3: tile j is in flight, tile j - 1's P V
        // is pending.  Barrier (every wave is done with tile j - 2), start
        // tile j + 1 into its stage, then tile j - 1's P V; the general steps
        // below continue with two tiles in flight.
        barrier_keep_dma();
        if (j + 1 < n_super) issue(st1, j + 1);
        pv16<T, true>(st2 + TILE, pw_prev, acc, lane);
      }
    } else {
      auto sync_full = [&](char* nxt, int j) __attribute__((always_inline)) {
        wait_vmem<2 * NCP>();
        barrier_keep_dma();
        issue_full(nxt, j + 2);
      };
      if (j_full > 0) {  // the first group: its first tile sets the offsets
        sync_full(st2, 0);
        compute_full(st0, 0, first);
        sync_full(st0, 1);
        compute_full(st1, 1, spec);
        sync_full(st1, 2);
        compute_full(st2, 2, spec);
        j = 3;
      }
      for (; j < j_full; j += 3) {
        sync_full(st2, j);
        compute_full(st0, j, spec);
        sync_full(st0, j + 1);
        compute_full(st1, j + 1, spec);
        sync_full(st1, j + 2);
        compute_full(st2, j + 2, spec);
      }
    }
    for (; j < n_super; j += 3) {
      sync(st2, j);
      compute(st0, j);
      if (j + 1 >= n_super) break;
      sync(st0, j + 1);
      compute(st1, j + 1);
      if (j + 2 >= n_super) break;
      sync(st1, j + 2);
      compute(st2, j + 2);
    }
  } else {
    // Two stages: wait for j, barrier, start j+1 into j-1's stage, compute j.
    auto sync = [&](char* nxt, int j) __attribute__((always_inline)) {
      wait_vmem<0>();
      barrier_keep_dma();
      if (j + 1 < n_super) issue(nxt, j + 1);
    };
    auto sync_full = [&](char* nxt, int j) __attribute__((always_inline)) {
      wait_vmem<0>();
      barrier_keep_dma();
      issue_full(nxt, j + 1);
    };
    if (j_full > 0) {  // the first pair: its first tile sets the offsets
      sync_full(st1, 0);
      compute_full(st0, 0, first);
      sync_full(st0, 1);
      compute_full(st1, 1, spec);
      j = 2;
    }
    for (; j < j_full; j += 2) {
      sync_full(st1, j);
      compute_full(st0, j, spec);
      sync_full(st0, j + 1);
      compute_full(st1, j + 1, spec);
    }
    for (; j < n_super; j += 2) {
      sync(st1, j);
      compute(st0, j);
      if (j + 1 >= n_super) break;
      sync(st0, j + 1);
      compute(st1, j + 1);
    }
  }
  if constexpr (!F32) l = lx[0];

  if constexpr (KS == 2) {
    // Merge the odd-tile waves' state into the even-tile waves (same query
    // rows, same register layout): with offsets m0, m1 and mt = max(m0, m1),
    // acc = acc0 2^(m0-mt) + acc1 2^(m1-mt), likewise l.  Stage 0 holds acc
    // as 16-byte quads [group][quad][lane]; stage 1 holds (m, l) per lane.
    // Every copy has completed (the last step waited for all of them).
    u32x4* racc = reinterpret_cast<u32x4*>(st0);
    u32x2* rml = reinterpret_cast<u32x2*>(st1);
    barrier_keep_dma();
    if (kh == 1) {
#pragma unroll
      for (int qd = 0; qd < 8; ++qd) {
        const f32x16& a = acc[qd >> 2];
        const int r = 4 * (qd & 3);
        const u32x4 w = {__float_as_uint(a[r]), __float_as_uint(a[r + 1]), __float_as_uint(a[r + 2]),
                         __float_as_uint(a[r + 3])};
        racc[(qg * 8 + qd) * 64 + lane] = w;
      }
      const u32x2 ml = {__float_as_uint(m), __float_as_uint(l)};
      rml[qg * 64 + lane] = ml;
    }
    barrier_keep_dma();
    if (kh == 1) return;
    const u32x2 ml1 = rml[qg * 64 + lane];
    const float m1 = __uint_as_float(ml1[0]);
    const float l1 = __uint_as_float(ml1[1]);
    const float mt = fmaxf(m, m1);
    const float a0 = (m == -INFINITY) ? 0.f : fast_exp2(m - mt);
    const float a1 = (m1 == -INFINITY) ? 0.f : fast_exp2(m1 - mt);
    l = l * a0 + l1 * a1;
    if constexpr (SPLIT) m = mt;  // the merged state's offset
#pragma unroll
    for (int qd = 0; qd < 8; ++qd) {
      const u32x4 w = racc[(qg * 8 + qd) * 64 + lane];
      f32x16& a = acc[qd >> 2];
      const int r = 4 * (qd & 3);
#pragma unroll
      for (int e = 0; e < 4; ++e) a[r + e] = a[r + e] * a0 + __uint_as_float(w[e]) * a1;
    }
  }

  // Epilogue: O = acc / l, rounded to T, for the rows this wave owns.  The
  // wave's 32-row tile is staged row-major in LDS (16-byte chunks XOR-swizzled
  // by row) and stored as whole rows, 64 lanes x 16 bytes per store: a store
  // of the accumulator layout directly would touch 32 rows per instruction
  // with 8- or 16-byte pieces.  Staging space: with one wave group, the stage
  // of the second-to-last key tile (every wave has passed it and no copy
  // targets it any more); with the key split, the wave's own part of the
  // merge area, which it has read.
  // The row's sum: 16-bit lanes hold the whole row's already (the matrix-core
  // row sums add both half-waves' keys); fp32 lanes hold their half's.
  const float lt = F32 ? l + other_half(l) : l;
  if constexpr (SPLIT) {
    // This key range's state of each valid row, one row per lane: fp32 acc
    // (its half of the columns per half-wave), and (m, l) from half-wave 0.
    if (qrow < row1) {
      const int64_t prow = ((int64_t)split * p.bh + head) * p.S_q + qrow;
      float* wa = p.ws_acc + prow * HEAD_DIM;
      if constexpr (F32) {
        // acc[dt] register 4g + e is column 16g + 8hf + 2e + dt
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
          const u32x4 w0 = {__float_as_uint(acc[0][4 * gq]), __float_as_uint(acc[1][4 * gq]),
                            __float_as_uint(acc[0][4 * gq + 1]), __float_as_uint(acc[1][4 * gq + 1])};
          const u32x4 w1 = {__float_as_uint(acc[0][4 * gq + 2]), __float_as_uint(acc[1][4 * gq + 2]),
                            __float_as_uint(acc[0][4 * gq + 3]), __float_as_uint(acc[1][4 * gq + 3])};
          *reinterpret_cast<u32x4*>(wa + 16 * gq + 8 * hf) = w0;
          *reinterpret_cast<u32x4*>(wa + 16 * gq + 8 * hf + 4) = w1;
        }
      } else {
        // acc[dt] register 4g + e is column 32dt + 8g + 4hf + e
#pragma unroll
        for (int dt = 0; dt < 2; ++dt)
#pragma unroll
          for (int gq = 0; gq < 4; ++gq) {
            const u32x4 w = {__float_as_uint(acc[dt][4 * gq]), __float_as_uint(acc[dt][4 * gq + 1]),
                             __float_as_uint(acc[dt][4 * gq + 2]), __float_as_uint(acc[dt][4 * gq + 3])};
            *reinterpret_cast<u32x4*>(wa + 32 * dt + 8 * gq + 4 * hf) = w;
          }
      }
      if (hf == 0) {
        const u32x2 ml = {__float_as_uint(m), __float_as_uint(lt)};
        *reinterpret_cast<u32x2*>(p.ws_ml + 2 * prow) = ml;
      }
    }
    return;
  }
  const float inv = (lt > 0.f) ? 1.0f / lt : 0.f;
  // Lane, column, half-wave and wave indices recomputed from an opaque copy
  // of the thread index: the staging offsets and store rows below equal
  // values the prologue computed, which the compiler would otherwise keep
  // live across the key loop (or spill, at three workgroups per CU).
  int tx = threadIdx.x;
  asm volatile("" : "+v"(tx));
  const int ln = tx & 63;
  const int ec = ln & 31, ehf = ln >> 5;
  // The output rows are stored with the non-temporal hint: this kernel never
  // reads them back, and the caches are better left to the K/V tiles other
  // workgroups are still reading (measured 0.5-3% faster on the short grids).
  auto store_row = [&](int row, int col, const u32x4& x) __attribute__((always_inline)) {
    if (wrow0 + row < row1)
      __builtin_nontemporal_store(x, reinterpret_cast<u32x4*>(oh + (int64_t)(wrow0 + row) * HEAD_DIM + col));
  };
  char* ot;
  if constexpr (KS == 1) {
    const int os = (n_super + 1) % 3;
    ot = (os == 0 ? st0 : os == 1 ? st1 : st2) + (tx >> 6) * (32 * ROWB);
  } else {
    ot = st0 + ((tx >> 6) % QG) * (8 * 64 * 16);
  }
  if constexpr (F32) {
    // acc[dt] row i = 8(r/4) + 4hf + r%4 is column d = 2i + dt: registers
    // 4g .. 4g+3 of both accumulators cover columns 16g + 8hf .. +7.
#pragma unroll
    for (int gq = 0; gq < 4; ++gq) {
      const int ch = 4 * gq + 2 * ehf;  // 16-byte chunk of columns 16g + 8hf .. +3
      u32x4 w0, w1;
      w0[0] = __float_as_uint(acc[0][4 * gq] * inv);
      w0[1] = __float_as_uint(acc[1][4 * gq] * inv);
      w0[2] = __float_as_uint(acc[0][4 * gq + 1] * inv);
      w0[3] = __float_as_uint(acc[1][4 * gq + 1] * inv);
      w1[0] = __float_as_uint(acc[0][4 * gq + 2] * inv);
      w1[1] = __float_as_uint(acc[1][4 * gq + 2] * inv);
      w1[2] = __float_as_uint(acc[0][4 * gq + 3] * inv);
      w1[3] = __float_as_uint(acc[1][4 * gq + 3] * inv);
      *reinterpret_cast<u32x4*>(ot + ec * 256 + 16 * (ch ^ (ec & 15))) = w0;
      *reinterpret_cast<u32x4*>(ot + ec * 256 + 16 * ((ch + 1) ^ (ec & 15))) = w1;
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) {  // rows 4k .. 4k+3
      const int row = 4 * k + ln / 16, ch = ln % 16;
      const u32x4 x = *reinterpret_cast<const u32x4*>(ot + row * 256 + 16 * (ch ^ (row & 15)));
      store_row(row, 4 * ch, x);
    }
  } else {
    typedef Half16<T> H;
    // acc[dt] register r is column 32dt + 8(r/4) + 4hf + r%4: registers 4g ..
    // 4g+3 are the half-chunk 8hf of 16-byte chunk 4dt + g.
#pragma unroll
    for (int dt = 0; dt < 2; ++dt) {
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        u32x2 w;
        w[0] = H::pack2(acc[dt][4 * gq] * inv, acc[dt][4 * gq + 1] * inv);
        w[1] = H::pack2(acc[dt][4 * gq + 2] * inv, acc[dt][4 * gq + 3] * inv);
        *reinterpret_cast<u32x2*>(ot + ec * 128 + 16 * ((4 * dt + gq) ^ (ec & 7)) + 8 * ehf) = w;
      }
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {  // rows 8k .. 8k+7
      const int row = 8 * k + ln / 8, ch = ln % 8;
      const u32x4 x = *reinterpret_cast<const u32x4*>(ot + row * 128 + 16 * (ch ^ (row & 7)));
      store_row(row, 8 * ch, x);
    }
  }
}

// Merge of the key ranges: row r's ranges hold (m_s, l_s, acc_s) with
// acc_s and l_s relative to 2^m_s; with M = max m_s the row is
// O = sum 2^(m_s - M) acc_s / sum 2^(m_s - M) l_s (a range in which the row
// saw no key has m_s = -inf and weight 0; a row that saw none at all gets
// zeros).  One thread per row and 16-byte chunk of its 64 columns.  The
// ranges are read MERGE_BATCH at a time, offsets, sums and accumulators
// together (indices clamped to the last range, the extra copies masked out),
// so that a batch costs one memory round trip; M is the largest offset seen
// so far, and a batch that raises it first rescales the running sums by
// 2^(M_old - M_new), the online-softmax update at range granularity.  With at
// most MERGE_BATCH ranges M is the maximum over all of them from the start.
constexpr int MERGE_THREADS = 256;
constexpr int MERGE_BATCH = 8;

template <typename T>
__global__ void __launch_bounds__(MERGE_THREADS) splitkv_merge_kernel(const float* __restrict__ ws_acc,
                                                                      const float* __restrict__ ws_ml,
                                                                      T* __restrict__ o, int64_t rows, int n_split) {
  const int64_t t = (int64_t)blockIdx.x * MERGE_THREADS + threadIdx.x;
  if (t >= rows * 16) return;
  const int64_t row = t >> 4;
  const int ch = (int)(t & 15);
  float mx = -INFINITY, L = 0.f, a[4] = {0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < n_split; s0 += MERGE_BATCH) {
    u32x2 ml[MERGE_BATCH];
    u32x4 x[MERGE_BATCH];
#pragma unroll
    for (int u = 0; u < MERGE_BATCH; ++u) {
      const int64_t pr = (int64_t)min(s0 + u, n_split - 1) * rows + row;
      ml[u] = *reinterpret_cast<const u32x2*>(ws_ml + 2 * pr);
      x[u] = *reinterpret_cast<const u32x4*>(ws_acc + pr * HEAD_DIM + 4 * ch);
    }
    float bx = -INFINITY;
#pragma unroll
    for (int u = 0; u < MERGE_BATCH; ++u) bx = fmaxf(bx, __uint_as_float(ml[u][0]));  // repeats change nothing
    if (bx > mx) {  // also the first batch with a visible key; -inf stays -inf
      const float r = (mx == -INFINITY) ? 0.f : fast_exp2(mx - bx);
      L *= r;
#pragma unroll
      for (int e = 0; e < 4; ++e) a[e] *= r;
      mx = bx;
    }
#pragma unroll
    for (int u = 0; u < MERGE_BATCH; ++u) {
      const float m = __uint_as_float(ml[u][0]);
      if (s0 + u >= n_split || m == -INFINITY) continue;
      const float w = fast_exp2(m - mx);
      L += w * __uint_as_float(ml[u][1]);
#pragma unroll
      for (int e = 0; e < 4; ++e) a[e] += w * __uint_as_float(x[u][e]);
    }
  }
  const float inv = (L > 0.f) ? 1.0f / L : 0.f;
  if constexpr (sizeof(T) == 4) {
    const u32x4 w = {__float_as_uint(a[0] * inv), __float_as_uint(a[1] * inv), __float_as_uint(a[2] * inv),
                     __float_as_uint(a[3] * inv)};
    *reinterpret_cast<u32x4*>(reinterpret_cast<float*>(o) + row * HEAD_DIM + 4 * ch) = w;
  } else {
    const u32x2 w = {Half16<T>::pack2(a[0] * inv, a[1] * inv), Half16<T>::pack2(a[2] * inv, a[3] * inv)};
    *reinterpret_cast<u32x2*>(o + row * HEAD_DIM + 4 * ch) = w;
  }
}

// The merge for more ranges than three batches: one workgroup per row,
// sixteen range groups x sixteen 16-byte chunks.  Group g folds ranges g, g + 16,
// g + 32, ... (MERGE_BATCH per memory round trip, the same running update as
// above), so up to 128 ranges take one round trip instead of one per batch;
// then the sixteen groups' (M_g, L_g, acc_g) of each chunk are combined
// through LDS with weights 2^(M_g - M).  Same result as the one-thread merge
// up to fp32 summation order.
constexpr int MERGE_GROUPS = 16;

template <typename T>
__global__ void __launch_bounds__(MERGE_GROUPS * 16) splitkv_merge_rows_kernel(const float* __restrict__ ws_acc,
                                                                              const float* __restrict__ ws_ml,
                                                                              T* __restrict__ o, int64_t rows,
                                                                              int n_split) {
  const int64_t row = blockIdx.x;
  const int ch = threadIdx.x & 15, g = threadIdx.x >> 4;
  float mx = -INFINITY, L = 0.f, a[4] = {0.f, 0.f, 0.f, 0.f};
  for (int s0 = g; s0 < n_split; s0 += MERGE_GROUPS * MERGE_BATCH) {
    u32x2 ml[MERGE_BATCH];
    u32x4 x[MERGE_BATCH];
#pragma unroll
    for (int u = 0; u < MERGE_BATCH; ++u) {
      const int sr = s0 + MERGE_GROUPS * u;
      const int64_t pr = (int64_t)(sr < n_split ? sr : g) * rows + row;  // g < n_split: a valid range
      ml[u] = *reinterpret_cast<const u32x2*>(ws_ml + 2 * pr);
      x[u] = *reinterpret_cast<const u32x4*>(ws_acc + pr * HEAD_DIM + 4 * ch);
    }
    float bx = -INFINITY;
#pragma unroll
    for (int u = 0; u < MERGE_BATCH; ++u)
      if (s0 + MERGE_GROUPS * u < n_split) bx = fmaxf(bx, __uint_as_float(ml[u][0]));
    if (bx > mx) {
      const float r = (mx == -INFINITY) ? 0.f : fast_exp2(mx - bx);
      L *= r;
#pragma unroll
      for (int e = 0; e < 4; ++e) a[e] *= r;
      mx = bx;
    }
#pragma unroll
    for (int u = 0; u < MERGE_BATCH; ++u) {
      const float m = __uint_as_float(ml[u][0]);
      if (s0 + MERGE_GROUPS * u >= n_split || m == -INFINITY) continue;
      const float w = fast_exp2(m - mx);
      L += w * __uint_as_float(ml[u][1]);
#pragma unroll
      for (int e = 0; e < 4; ++e) a[e] += w * __uint_as_float(x[u][e]);
    }
  }
  __shared__ float part[MERGE_GROUPS][16][6];
  part[g][ch][0] = mx;
  part[g][ch][1] = L;
#pragma unroll
  for (int e = 0; e < 4; ++e) part[g][ch][2 + e] = a[e];
  __syncthreads();
  if (g != 0) return;
  float M = -INFINITY;
#pragma unroll
  for (int h = 0; h < MERGE_GROUPS; ++h) M = fmaxf(M, part[h][ch][0]);
  L = 0.f;
#pragma unroll
  for (int e = 0; e < 4; ++e) a[e] = 0.f;
#pragma unroll
  for (int h = 0; h < MERGE_GROUPS; ++h) {
    const float mh = part[h][ch][0];
    if (mh == -INFINITY) continue;  // a group with no visible key (or no range)
    const float w = fast_exp2(mh - M);
    L += w * part[h][ch][1];
#pragma unroll
    for (int e = 0; e < 4; ++e) a[e] += w * part[h][ch][2 + e];
  }
  const float inv = (L > 0.f) ? 1.0f / L : 0.f;
  if constexpr (sizeof(T) == 4) {
    const u32x4 w = {__float_as_uint(a[0] * inv), __float_as_uint(a[1] * inv), __float_as_uint(a[2] * inv),
                     __float_as_uint(a[3] * inv)};
    *reinterpret_cast<u32x4*>(reinterpret_cast<float*>(o) + row * HEAD_DIM + 4 * ch) = w;
  } else {
    const u32x2 w = {Half16<T>::pack2(a[0] * inv, a[1] * inv), Half16<T>::pack2(a[2] * inv, a[3] * inv)};
    *reinterpret_cast<u32x2*>(o + row * HEAD_DIM + 4 * ch) = w;
  }
}

}  // namespace

// The split-key partial states of attn_fwd_splitkv_noalloc: device memory of
// the library itself, so that entry point allocates nothing.  Every GPU the
// library runs on holds its own copy until the process ends, and every call on
// that GPU reuses it (the contents of the previous call stay; the split
// kernels write every state the merge reads, so nothing needs clearing).
static __device__ __align__(256) unsigned char scratch[ATTN_NOALLOC_SCRATCH_BYTES];

namespace {

// Device address of `scratch` on each device, looked up once per device with
// that device current (the array's name is a host-side stand-in, not a device
// address, so only this pointer ever reaches a kernel).
std::mutex g_scratch_mu;
std::atomic<void*> g_scratch[64];

int scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return ATTN_E_DEVICE;
  if (dev < 64) {
    void* p = g_scratch[dev].load(std::memory_order_acquire);
    if (p) {
      *out = p;
      return ATTN_OK;
    }
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  void* p = dev < 64 ? g_scratch[dev].load(std::memory_order_acquire) : nullptr;
  if (!p) {
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return ATTN_E_HIP;
    if (dev < 64) g_scratch[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return ATTN_OK;
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------
int validate(const void* q, const void* k, const void* v, void* o, int B, int H, int S_q, int S_kv,
             int D_h, int causal, float scale, int dtype, int chunk, int kv_len) {
  if (!q || !k || !v || !o) return ATTN_E_NULL;
  if (B < 1 || H < 1 || S_q < 1 || S_kv < 1 || D_h != HEAD_DIM) return ATTN_E_SHAPE;
  if (dtype != ATTN_F32 && dtype != ATTN_F16 && dtype != ATTN_BF16) return ATTN_E_DTYPE;
  uint32_t sbits;
  std::memcpy(&sbits, &scale, 4);
  if ((sbits & 0x7f800000u) == 0x7f800000u) return ATTN_E_SCALE;  // NaN or infinity
  if (chunk < 1 || kv_len < 1 || kv_len > S_kv) return ATTN_E_CHUNK;
  if (causal && S_q > kv_len) return ATTN_E_CAUSAL;
  // sizes: elements and bytes fit in int64; the grid fits in 2^31 - 1
  const int64_t bh = (int64_t)B * H;
  if (bh > (int64_t)INT32_MAX) return ATTN_E_SHAPE;
  const int64_t esz = dtype == ATTN_F32 ? 4 : 2;
  const int64_t lim = INT64_MAX / (HEAD_DIM * esz);
  if ((int64_t)S_q > lim / bh || (int64_t)S_kv > lim / bh) return ATTN_E_SHAPE;
  // tile copies address one head of K/V with 32-bit byte offsets
  if ((int64_t)S_kv * HEAD_DIM * esz > (int64_t)UINT32_MAX) return ATTN_E_SHAPE;
  const int64_t n_win = ((int64_t)S_q + chunk - 1) / chunk;
  const int64_t tiles = n_win * (((int64_t)std::min(chunk, S_q) + BM - 1) / BM);
  if (tiles * bh > (int64_t)INT32_MAX) return ATTN_E_SHAPE;
  const uintptr_t mis = ((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o) & 15u;
  if (mis) return ATTN_E_ALIGN;
  const uint64_t nq = (uint64_t)bh * S_q * HEAD_DIM * esz;
  const uint64_t nkv = (uint64_t)bh * S_kv * HEAD_DIM * esz;
  if (ranges_overlap(o, nq, q, nq) || ranges_overlap(o, nq, k, nkv) || ranges_overlap(o, nq, v, nkv))
    return ATTN_E_OVERLAP;
  return ATTN_OK;
}

Sched make_sched(int B, int H, int S_q, int chunk, int kv_len, int causal, int bm) {
  Sched s;
  s.bm = bm;
  s.tile_major = causal && kv_len <= TILE_MAJOR_MAX_KV;
  s.S_q = S_q;
  s.chunk = std::min(chunk, S_q);
  s.n_win = (S_q + s.chunk - 1) / s.chunk;
  s.tf = (s.chunk + bm - 1) / bm;
  const int last_rows = S_q - (s.n_win - 1) * s.chunk;
  s.tl = (last_rows + bm - 1) / bm;
  const int bh = B * H;
  s.groups = (bh % 8 == 0) ? 8 : 1;
  s.heads = bh / s.groups;
  return s;
}

template <typename T, int KS, bool VARLEN, bool SPLIT, int QG>
void launch_kernel_v(const Params<T>& p, int grid, int causal, hipStream_t stream) {
  if (causal)
    hipLaunchKernelGGL((attn_fwd_kernel<T, true, KS, VARLEN, SPLIT, QG>), dim3(grid), dim3(64 * QG * KS), 0,
                       stream, p);
  else
    hipLaunchKernelGGL((attn_fwd_kernel<T, false, KS, VARLEN, SPLIT, QG>), dim3(grid), dim3(64 * QG * KS), 0,
                       stream, p);
}

template <typename T, int KS, int QG = 4>
void launch_kernel(const Params<T>& p, int grid, int causal, hipStream_t stream) {
  if (p.kv_lens)
    launch_kernel_v<T, KS, true, false, QG>(p, grid, causal, stream);
  else
    launch_kernel_v<T, KS, false, false, QG>(p, grid, causal, stream);
}

// Query rows per workgroup of an attn_fwd / attn_fwd_chunked / attn_fwd_varlen
// launch, and whether the keys are split between two wave groups.  Few
// 128-row query tiles (at most two per CU): split each tile's key range
// between two wave groups so every SIMD runs two waves on half the key chain.
// 16-bit types then take 64-row tiles (four waves: 2 query groups x 2 key
// halves, two workgroups per CU) where the finer grain balances the CUs:
// causal grids below two 128-row tiles per CU (their tiles differ in length),
// and other grids whose last round of 128-row tiles would fill at most half
// the CUs.  Elsewhere a CU running two 64-row workgroups is slower than one
// eight-wave workgroup on the same rows (each loads all K/V for half the
// rows).  fp32 takes them only while the 64-row grid still gives every
// workgroup a CU of its own (its two LDS stages fill 128 KB): each SIMD then
// runs one wave instead of two.  The choice depends on B, H, S_q, causal, the
// type and the CU count only, never on the window size, so chunked and
// unchunked calls sum in the same order.  At most 32 query rows per head
// (decode steps): one 32-row query group per workgroup, its keys split
// between two waves, so that no wave of the workgroup idles.
void launch_shape(int B, int H, int S_q, int causal, int dtype, int n_cu, int& rows, int& ks) {
  if (S_q <= 32) {
    rows = 32;
    ks = 2;
    return;
  }
  const int64_t tiles = (int64_t)B * H * ((S_q + BM - 1) / BM);
  ks = tiles <= 2 * (int64_t)n_cu ? 2 : 1;
  const int64_t last = tiles % n_cu;  // 128-row tiles in a last, partial round
  const bool fine = dtype == ATTN_F32 ? 2 * tiles <= (int64_t)n_cu
                                      : ks == 2 && (causal ? tiles < 2 * (int64_t)n_cu
                                                           : last != 0 && 2 * last <= (int64_t)n_cu);
  rows = fine ? 64 : BM;
}

template <typename T>
int launch_typed(const void* q, const void* k, const void* v, void* o, int B, int H, int S_q, int S_kv,
                 int causal, float scale, hipStream_t stream, int chunk, int kv_len, int n_cu,
                 const int* kv_lens = nullptr, int n_split = 1, void* ws = nullptr) {
  Params<T> p;
  p.q = static_cast<const T*>(q);
  p.k = static_cast<const T*>(k);
  p.v = static_cast<const T*>(v);
  p.o = static_cast<T*>(o);
  p.q_head_stride = (int64_t)S_q * HEAD_DIM;
  p.kv_head_stride = (int64_t)S_kv * HEAD_DIM;
  p.S_q = S_q;
  p.kv_len = kv_len;
  p.kv_lens = kv_lens;
  p.H = H;
  p.S_kv = S_kv;
  p.ws_acc = nullptr;
  p.ws_ml = nullptr;
  p.split_span = 0;
  p.bh = B * H;
  // |scale| * log2(e), at least 1e-30 so that a masked score (-inf) always
  // exponentiates to 0; for scale = 0 every visible probability is still
  // exp2(~1e-27) = 1 exactly in fp32.
  p.c = (float)std::max(std::fabs((double)scale) * 1.4426950408889634, 1e-30);
  p.q_flip = (scale < 0.f) ? (sizeof(T) == 4 ? 0x80000000u : 0x80008000u) : 0u;
  int rows = BM, ks = 1;
  if (n_split == 1) {
    launch_shape(B, H, S_q, causal, sizeof(T) == 4 ? ATTN_F32 : ATTN_BF16, n_cu, rows, ks);
  } else if (S_q <= 32) {  // decode steps: 32-row tiles, keys split between two waves in each range
    rows = 32;
    ks = 2;
  }
  p.s = make_sched(B, H, S_q, chunk, kv_len, causal, rows);
  const int grid = p.s.groups * p.s.heads * (p.s.tl + (p.s.n_win - 1) * p.s.tf);
  p.base_grid = grid;
  if (n_split > 1) {
    // Split the keys into n_split ranges of whole 64-key tiles; the four-wave
    // workgroup runs every range (several per CU keep more tile copies in
    // flight than one eight-wave workgroup), or for at most 32 query rows the
    // two-wave 32-row workgroup (each wave half of the range).  Ranges past
    // the last tile are empty.
    const int kv_tiles = (kv_len + BN - 1) / BN;
    const int per = (kv_tiles + n_split - 1) / n_split;
    p.split_span = per * BN;
    p.ws_acc = static_cast<float*>(ws);
    const int64_t rows = (int64_t)B * H * S_q;
    p.ws_ml = p.ws_acc + (int64_t)n_split * rows * HEAD_DIM;
    if (rows == 32)
      launch_kernel_v<T, 2, false, true, 1>(p, grid * n_split, causal, stream);
    else
      launch_kernel_v<T, 1, false, true, 4>(p, grid * n_split, causal, stream);
    if (hipGetLastError() != hipSuccess) return ATTN_E_HIP;
    if (n_split > 3 * MERGE_BATCH && rows <= (int64_t)INT32_MAX) {  // more than three batches per row
      hipLaunchKernelGGL((splitkv_merge_rows_kernel<T>), dim3((unsigned)rows), dim3(MERGE_GROUPS * 16), 0, stream,
                         p.ws_acc, p.ws_ml, static_cast<T*>(o), rows, n_split);
    } else {
      const int64_t mblocks = (rows * 16 + MERGE_THREADS - 1) / MERGE_THREADS;
      hipLaunchKernelGGL((splitkv_merge_kernel<T>), dim3((unsigned)mblocks), dim3(MERGE_THREADS), 0, stream,
                         p.ws_acc, p.ws_ml, static_cast<T*>(o), rows, n_split);
    }
    return hipGetLastError() == hipSuccess ? ATTN_OK : ATTN_E_HIP;
  }
  if (ks == 1)
    launch_kernel<T, 1>(p, grid, causal, stream);
  else if (rows == 32)
    launch_kernel<T, 2, 1>(p, grid, causal, stream);
  else if (rows == 64)
    launch_kernel<T, 2, 2>(p, grid, causal, stream);
  else
    launch_kernel<T, 2>(p, grid, causal, stream);
  return hipGetLastError() == hipSuccess ? ATTN_OK : ATTN_E_HIP;
}

// ---------------------------------------------------------------------------
// K/V cache append (streaming use of the chunked entry point)
// ---------------------------------------------------------------------------
// Head g's n_new new rows are one contiguous segment of the source, and land
// contiguously at row kv_len of that head's cache: a plain copy, 16 bytes per
// lane per step, K and V in the same launch.  blockIdx.x walks the segment in
// blocks of APPEND_UNITS 16-byte units, blockIdx.y (and the loop) the heads.
constexpr int APPEND_THREADS = 256;
constexpr int APPEND_UNITS = APPEND_THREADS * 4;  // 16-byte units per block and head

__global__ void __launch_bounds__(APPEND_THREADS) kv_append_kernel(char* kc, char* vc, const char* kn, const char* vn,
                                                                  int64_t heads, int64_t head_units,
                                                                  int64_t cache_head_bytes, int64_t dst_off) {
  const int64_t u0 = (int64_t)blockIdx.x * APPEND_UNITS + threadIdx.x;
  for (int64_t g = blockIdx.y; g < heads; g += gridDim.y) {
    const int64_t src = g * head_units * 16;
    const int64_t dst = g * cache_head_bytes + dst_off;
#pragma unroll
    for (int r = 0; r < APPEND_UNITS / APPEND_THREADS; ++r) {
      const int64_t u = u0 + r * APPEND_THREADS;
      if (u < head_units) {
        const u32x4 k = *reinterpret_cast<const u32x4*>(kn + src + u * 16);
        const u32x4 v = *reinterpret_cast<const u32x4*>(vn + src + u * 16);
        *reinterpret_cast<u32x4*>(kc + dst + u * 16) = k;
        *reinterpret_cast<u32x4*>(vc + dst + u * 16) = v;
      }
    }
  }
}

}  // namespace

extern "C" int attn_kv_append(void* k_cache, void* v_cache, const void* k_new, const void* v_new, int B, int H,
                              int S_cap, int kv_len, int n_new, int D_h, int dtype, void* stream) {
  if (!k_cache || !v_cache || !k_new || !v_new) return ATTN_E_NULL;
  if (B < 1 || H < 1 || S_cap < 1 || n_new < 1 || kv_len < 0 || D_h != HEAD_DIM) return ATTN_E_SHAPE;
  if ((int64_t)kv_len + n_new > S_cap) return ATTN_E_SHAPE;
  if (dtype != ATTN_F32 && dtype != ATTN_F16 && dtype != ATTN_BF16) return ATTN_E_DTYPE;
  const int64_t bh = (int64_t)B * H;
  const int64_t row_bytes = (int64_t)HEAD_DIM * (dtype == ATTN_F32 ? 4 : 2);
  if ((int64_t)S_cap > INT64_MAX / row_bytes / bh) return ATTN_E_SHAPE;
  const uintptr_t mis = ((uintptr_t)k_cache | (uintptr_t)v_cache | (uintptr_t)k_new | (uintptr_t)v_new) & 15u;
  if (mis) return ATTN_E_ALIGN;
  const uint64_t nc = (uint64_t)bh * S_cap * row_bytes, nn = (uint64_t)bh * n_new * row_bytes;
  if (ranges_overlap(k_cache, nc, v_cache, nc) || ranges_overlap(k_cache, nc, k_new, nn) ||
      ranges_overlap(k_cache, nc, v_new, nn) || ranges_overlap(v_cache, nc, k_new, nn) ||
      ranges_overlap(v_cache, nc, v_new, nn))
    return ATTN_E_OVERLAP;
  int n_cu = 0;
  const int dv = check_device(&n_cu);
  if (dv != ATTN_OK) return dv;
  const int64_t head_units = (int64_t)n_new * row_bytes / 16;
  const int64_t bx = (head_units + APPEND_UNITS - 1) / APPEND_UNITS;
  if (bx > INT32_MAX) return ATTN_E_SHAPE;
  const int by = (int)std::min<int64_t>(bh, 65535);
  hipLaunchKernelGGL(kv_append_kernel, dim3((unsigned)bx, (unsigned)by), dim3(APPEND_THREADS), 0,
                     static_cast<hipStream_t>(stream), static_cast<char*>(k_cache), static_cast<char*>(v_cache),
                     static_cast<const char*>(k_new), static_cast<const char*>(v_new), bh, head_units,
                     (int64_t)S_cap * row_bytes, (int64_t)kv_len * row_bytes);
  return hipGetLastError() == hipSuccess ? ATTN_OK : ATTN_E_HIP;
}

extern "C" int attn_fwd_chunked(const void* q, const void* k, const void* v, void* o, int B, int H, int S_q,
                                int S_kv, int D_h, int causal, float scale, int dtype, void* stream,
                                int chunk, int kv_len) {
  const int st = validate(q, k, v, o, B, H, S_q, S_kv, D_h, causal, scale, dtype, chunk, kv_len);
  if (st != ATTN_OK) return st;
  int n_cu = 0;
  const int dv = check_device(&n_cu);
  if (dv != ATTN_OK) return dv;
  hipStream_t s = static_cast<hipStream_t>(stream);
  switch (dtype) {
    case ATTN_F32:
      return launch_typed<float>(q, k, v, o, B, H, S_q, S_kv, causal, scale, s, chunk, kv_len, n_cu);
    case ATTN_F16:
      return launch_typed<_Float16>(q, k, v, o, B, H, S_q, S_kv, causal, scale, s, chunk, kv_len, n_cu);
    default:
      return launch_typed<__bf16>(q, k, v, o, B, H, S_q, S_kv, causal, scale, s, chunk, kv_len, n_cu);
  }
}

extern "C" int attn_fwd(const void* q, const void* k, const void* v, void* o, int B, int H, int S_q, int S_kv,
                        int D_h, int causal, float scale, int dtype, void* stream) {
  return attn_fwd_chunked(q, k, v, o, B, H, S_q, S_kv, D_h, causal, scale, dtype, stream, S_q, S_kv);
}

extern "C" int attn_fwd_varlen(const void* q, const void* k, const void* v, void* o, int B, int H, int S_q,
                               int S_kv, int D_h, int causal, float scale, int dtype, void* stream,
                               const int* kv_lens) {
  if (!kv_lens) return ATTN_E_NULL;
  if ((uintptr_t)kv_lens & 3u) return ATTN_E_ALIGN;
  // Checked as a non-causal call over the whole cache: with per-sequence
  // lengths a causal row may see no key (it gets zeros).
  const int st = validate(q, k, v, o, B, H, S_q, S_kv, D_h, 0, scale, dtype, S_q, S_kv);
  if (st != ATTN_OK) return st;
  int n_cu = 0;
  const int dv = check_device(&n_cu);
  if (dv != ATTN_OK) return dv;
  hipStream_t s = static_cast<hipStream_t>(stream);
  switch (dtype) {
    case ATTN_F32:
      return launch_typed<float>(q, k, v, o, B, H, S_q, S_kv, causal, scale, s, S_q, S_kv, n_cu, kv_lens);
    case ATTN_F16:
      return launch_typed<_Float16>(q, k, v, o, B, H, S_q, S_kv, causal, scale, s, S_q, S_kv, n_cu, kv_lens);
    default:
      return launch_typed<__bf16>(q, k, v, o, B, H, S_q, S_kv, causal, scale, s, S_q, S_kv, n_cu, kv_lens);
  }
}

extern "C" int attn_splitkv_workspace_bytes(int B, int H, int S_q, int n_split, size_t* bytes) {
  if (!bytes || B < 1 || H < 1 || S_q < 1) return ATTN_E_SHAPE;
  if (n_split < 1 || n_split > MAX_SPLIT) return ATTN_E_SPLIT;
  if (n_split == 1) {
    *bytes = 0;
    return ATTN_OK;
  }
  const int64_t rows = (int64_t)B * H * S_q;
  const int64_t per_row = (HEAD_DIM + 2) * 4;  // fp32 acc, then (m, l)
  if (rows > INT64_MAX / per_row / n_split) return ATTN_E_SHAPE;
  *bytes = (size_t)(rows * per_row * n_split);
  return ATTN_OK;
}

extern "C" int attn_splitkv_choose(int B, int H, int S_q, int kv_len, int n_cu, int* n_split) {
  if (!n_split || B < 1 || H < 1 || S_q < 1 || kv_len < 1 || n_cu < 1) return ATTN_E_SHAPE;
  const int64_t tiles = (int64_t)B * H * ((S_q + BM - 1) / BM);
  const int64_t kv_tiles = (kv_len + BN - 1) / BN;
  // Measured on decode steps and short prefill windows: about one workgroup
  // per CU (rows with many ranges merge them in parallel, so a single head
  // against a long cache takes as many ranges as there are CUs); two ranges
  // from one to two query tiles per CU.
  int64_t n = 1;
  if (kv_tiles >= SPLIT_MIN_KV_TILES) {
    if (tiles < n_cu) {
      n = (n_cu + tiles - 1) / tiles;  // about n_cu workgroups
      n = std::min<int64_t>(n, kv_tiles / 2);  // each range keeps at least two key tiles
    } else if (tiles < 2 * (int64_t)n_cu) {
      n = 2;
    }
    n = std::max<int64_t>(1, std::min<int64_t>(n, MAX_SPLIT));
  }
  *n_split = (int)n;
  return ATTN_OK;
}

namespace {

// attn_fwd_splitkv's checks and launches for a workspace the caller brings
// (own_ws = false: null, misaligned, short or overlapping workspaces are
// rejected) or the library's scratch array (own_ws = true: the array's
// device address, looked up after the argument checks).
int splitkv_impl(const void* q, const void* k, const void* v, void* o, int B, int H, int S_q, int S_kv, int D_h,
                 int causal, float scale, int dtype, void* stream, int kv_len, int n_split, void* workspace,
                 size_t workspace_bytes, bool own_ws) {
  const int st = validate(q, k, v, o, B, H, S_q, S_kv, D_h, causal, scale, dtype, S_q, kv_len);
  if (st != ATTN_OK) return st;
  size_t need = 0;
  const int ws = attn_splitkv_workspace_bytes(B, H, S_q, n_split, &need);
  if (ws != ATTN_OK) return ws;
  const Sched sc = make_sched(B, H, S_q, S_q, kv_len, causal, BM);
  const int64_t grid = (int64_t)sc.groups * sc.heads * sc.tl;
  const int64_t rows = (int64_t)B * H * S_q;
  if (grid * n_split > INT32_MAX || (rows * 16 + MERGE_THREADS - 1) / MERGE_THREADS > INT32_MAX) return ATTN_E_SPLIT;
  if (own_ws) {
    if (need > ATTN_NOALLOC_SCRATCH_BYTES) return ATTN_E_WORKSPACE;
  } else if (n_split > 1) {
    if (!workspace || ((uintptr_t)workspace & 15u) || workspace_bytes < need) return ATTN_E_WORKSPACE;
    const uint64_t esz = dtype == ATTN_F32 ? 4 : 2;
    const uint64_t nq = (uint64_t)rows * HEAD_DIM * esz, nkv = (uint64_t)B * H * S_kv * HEAD_DIM * esz;
    if (ranges_overlap(workspace, need, q, nq) || ranges_overlap(workspace, need, o, nq) ||
        ranges_overlap(workspace, need, k, nkv) || ranges_overlap(workspace, need, v, nkv))
      return ATTN_E_WORKSPACE;
  }
  int n_cu = 0;
  const int dv = check_device(&n_cu);
  if (dv != ATTN_OK) return dv;
  if (own_ws && n_split > 1) {
    const int sp = scratch_address(&workspace);
    if (sp != ATTN_OK) return sp;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  switch (dtype) {
    case ATTN_F32:
      return launch_typed<float>(q, k, v, o, B, H, S_q, S_kv, causal, scale, s, S_q, kv_len, n_cu, nullptr, n_split,
                                 workspace);
    case ATTN_F16:
      return launch_typed<_Float16>(q, k, v, o, B, H, S_q, S_kv, causal, scale, s, S_q, kv_len, n_cu, nullptr,
                                    n_split, workspace);
    default:
      return launch_typed<__bf16>(q, k, v, o, B, H, S_q, S_kv, causal, scale, s, S_q, kv_len, n_cu, nullptr,
                                  n_split, workspace);
  }
}

}  // namespace

extern "C" int attn_fwd_splitkv(const void* q, const void* k, const void* v, void* o, int B, int H, int S_q,
                                int S_kv, int D_h, int causal, float scale, int dtype, void* stream, int kv_len,
                                int n_split, void* workspace, size_t workspace_bytes) {
  return splitkv_impl(q, k, v, o, B, H, S_q, S_kv, D_h, causal, scale, dtype, stream, kv_len, n_split, workspace,
                      workspace_bytes, false);
}

extern "C" int attn_fwd_splitkv_noalloc(const void* q, const void* k, const void* v, void* o, int B, int H,
                                        int S_q, int S_kv, int D_h, int causal, float scale, int dtype,
                                        void* stream, int kv_len, int n_split) {
  return splitkv_impl(q, k, v, o, B, H, S_q, S_kv, D_h, causal, scale, dtype, stream, kv_len, n_split, nullptr, 0,
                      true);
}

extern "C" int attn_sched_rows(int B, int H, int S_q, int causal, int dtype, int n_cu, int* rows,
                               int* key_split) {
  if (B < 1 || H < 1 || S_q < 1 || n_cu < 1 || !rows || !key_split) return ATTN_E_SHAPE;
  if (dtype != ATTN_F32 && dtype != ATTN_F16 && dtype != ATTN_BF16) return ATTN_E_DTYPE;
  launch_shape(B, H, S_q, causal, dtype, n_cu, *rows, *key_split);
  return ATTN_OK;
}

extern "C" int attn_sched_grid(int B, int H, int S_q, int chunk, int kv_len, int causal, int rows, int* grid) {
  if (B < 1 || H < 1 || S_q < 1 || chunk < 1 || kv_len < 1 || !grid) return ATTN_E_SHAPE;
  if (rows != 32 && rows != 64 && rows != BM) return ATTN_E_SHAPE;
  const int64_t bh = (int64_t)B * H;
  const int64_t n_win = ((int64_t)S_q + chunk - 1) / chunk;
  const int64_t tiles = n_win * (((int64_t)std::min(chunk, S_q) + rows - 1) / rows);
  if (bh > (int64_t)INT32_MAX || tiles * bh > (int64_t)INT32_MAX) return ATTN_E_SHAPE;
  const Sched s = make_sched(B, H, S_q, chunk, kv_len, causal, rows);
  *grid = s.groups * s.heads * (s.tl + (s.n_win - 1) * s.tf);
  return ATTN_OK;
}

extern "C" int attn_sched_tile(int B, int H, int S_q, int chunk, int kv_len, int causal, int rows, int block,
                               int* head, int* row0, int* row1) {
  int grid = 0;
  const int st = attn_sched_grid(B, H, S_q, chunk, kv_len, causal, rows, &grid);
  if (st != ATTN_OK) return st;
  if (block < 0 || block >= grid || !head || !row0 || !row1) return ATTN_E_SHAPE;
  decode_tile(make_sched(B, H, S_q, chunk, kv_len, causal, rows), block, *head, *row0, *row1);
  return ATTN_OK;
}

extern "C" const char* attn_strerror(int status) {
  switch (status) {
    case ATTN_OK: return "success";
    case ATTN_E_NULL: return "null tensor pointer";
    case ATTN_E_SHAPE: return "invalid shape (B, H, S_q, S_kv must be >= 1, D_h must be 64, sizes must fit)";
    case ATTN_E_DTYPE: return "unknown dtype (expected ATTN_F32, ATTN_F16 or ATTN_BF16)";
    case ATTN_E_SCALE: return "scale is not finite";
    case ATTN_E_CAUSAL: return "causal attention needs S_q <= kv_len";
    case ATTN_E_CHUNK: return "chunk must be >= 1 and kv_len in [1, S_kv]";
    case ATTN_E_ALIGN: return "tensor base pointer not 16-byte aligned";
    case ATTN_E_OVERLAP: return "output overlaps an input";
    case ATTN_E_DEVICE: return "current HIP device missing or not gfx950";
    case ATTN_E_HIP: return "HIP runtime error at kernel launch";
    case ATTN_E_SPLIT: return "n_split outside [1, 1024], or the split grid is too large";
    case ATTN_E_WORKSPACE: return "workspace null, not 16-byte aligned, too small, or overlapping a tensor";
    default: return "unknown attn status";
  }
}
