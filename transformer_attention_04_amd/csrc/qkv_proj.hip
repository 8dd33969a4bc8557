// qkv_proj.hip -- fused Q/K/V projection for AMD Instinct MI355X (gfx950).
//
// The step upstream of attention: the layer input x [B, S, d] times the three
// projection weights stacked as one linear-layer weight W [3d, d] (rows q,
// then k, then v; 64 rows per head), plus an optional bias, as ONE matrix
// product whose epilogue writes each 64-column head group straight into the
// [B, H, S, 64] layout the attention kernels read (page "Roofline", sections
// "What it does" and "How we built it": the Q/K/V projections fused into one
// larger kernel).  No [B*S, 3d] intermediate exists.
//
// Work decomposition
//   C = x W^T with M = B*S rows, N = 3d columns, K = d.  A workgroup of 8
//   wavefronts owns a PM x PN = 256 x 256 tile of C and walks K in stages of
//   PK = 64: per stage it copies the tile's 256 rows of x and 256 rows of W
//   (128 bytes each) straight into LDS (global_load_lds_dwordx4, 16-byte
//   chunks XOR-swizzled per row, the layout of the attention kernels' K
//   tiles), two stages in flight-and-compute.  Both operands are contiguous
//   in K, so the MFMA computes C^T = W x^T: lane l of a 32 x 32 block owns
//   one row of C (row l % 32) and 16 of its columns; the accumulators start
//   from the bias, and the epilogue goes through LDS so that every store is a
//   whole 16-byte piece of an output row.  Wave (wm, wn) = (wave % 4, wave / 4)
//   owns rows 64 wm .. +63 and columns 128 wn .. +127 of the tile: 2 x 4
//   blocks of v_mfma_f32_32x32x16_{bf16,f16}, fp32 accumulation (128
//   accumulator registers of the 256 each of the two waves per SIMD has).
//   Tiles are dealt to the XCDs (workgroups go round-robin over the 8 XCDs)
//   as 8 rectangular parts of the tile grid: cg column groups by 8 / cg row
//   groups.  Inside a part the tiles run row block major, so the 32
//   workgroups an XCD holds at once cover about 32 / c row blocks and c
//   column tiles (c = column tiles per part) and read each of those x and W
//   blocks once from beyond the XCD's L2 while they walk K together; the
//   host picks the cg that makes 32 / c + c, the blocks fetched per such
//   round, smallest.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "attn.h"
#include "gfx950.h"
#include "host_common.h"

namespace {

constexpr int PM = 256;                     // rows of x per workgroup
constexpr int PN = 256;                     // rows of W (columns of C) per workgroup
constexpr int PK = 64;                      // K per stage (one 128-byte row segment)
constexpr int PTHREADS = 512;               // 8 wavefronts, two per SIMD
constexpr int PROWB = PK * 2;               // bytes per staged row
constexpr int PHALF = PM * PROWB;           // 32 KB: one stage of x (or of W)
// LDS: x stage 0 | x stage 1 | W stage 0 | W stage 1.  Every operand read is
// a per-lane base plus a constant below 64 KB (stage, block), which the
// ds_read instruction takes as its immediate offset.
constexpr int PLDS = 4 * PHALF;
static_assert(PM == PN, "x and W stages share one size");

template <typename T>
struct ProjParams {
  const T* x;     // [M, K]
  const T* w;     // [N, K]
  const T* bias;  // [N] or null
  T* out[3];      // q, k, v: [B, H, S, 64]
  int M, N, K;    // B*S, 3d, d
  int S, H;
  int tiles_n;    // column tiles
  int tiles;      // total tiles
  int cg;         // column groups of the XCD parts (1, 2, 4 or 8), or 0: plain row-major order
  int prows;      // row blocks per part
  int pcols;      // column tiles per part
};

template <typename T>
__global__ void __launch_bounds__(PTHREADS, 1) qkv_proj_kernel(ProjParams<T> p) {
  typedef Half16<T> H16;
  typedef typename H16::vec8 vec8;
  __shared__ __attribute__((aligned(16))) char lds[PLDS];

  // Tile of this workgroup: block b runs on XCD x = b % 8 as that XCD's
  // i = b / 8-th tile; part x is column group x % cg, row group x / cg.
  int mt, nt;
  if (p.cg) {
    const int x = blockIdx.x & 7, i = blockIdx.x >> 3;
    const int ri = i / p.pcols;
    mt = (x / p.cg) * p.prows + ri;
    nt = (x % p.cg) * p.pcols + (i - ri * p.pcols);
  } else {
    mt = blockIdx.x / p.tiles_n;
    nt = blockIdx.x - mt * p.tiles_n;
  }
  const int m0 = mt * PM, n0 = nt * PN;

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int c = lane & 31, hf = lane >> 5;
  const int wm = wave & 3, wn = wave >> 2;

  // Copies: wave w fills staged rows 32w .. +31 of x and of W, 8 rows per
  // instruction; lane l lands in row r = 32w + 8i + l/8 at physical chunk
  // l % 8 and fetches the logical chunk the row's swizzle maps there: with
  // swizzle (r & 7) ^ ((r >> 3) & 1) = (l / 8) ^ (i & 1) that is chunk
  // (l % 8) ^ (l / 8) ^ (i & 1).  Rows past the matrix end re-read its last
  // row (finite data, never stored).  The eight source addresses of stage 0
  // are kept (16 registers); stage kt adds kt * 128 bytes.
  const char* src[8];
  {
    const int crow = 32 * wave + lane / 8;
    const int cch = (lane % 8) ^ (lane / 8);
    const char* const xb = reinterpret_cast<const char*>(p.x);
    const char* const wb = reinterpret_cast<const char*>(p.w);
    const int64_t rowb = (int64_t)p.K * 2;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = crow + 8 * i;
      const int col = 16 * (cch ^ (i & 1));
      src[2 * i] = xb + min(m0 + r, p.M - 1) * rowb + col;
      src[2 * i + 1] = wb + min(n0 + r, p.N - 1) * rowb + col;
    }
  }
  const uint32_t wdst = __builtin_amdgcn_readfirstlane((uint32_t)(32 * wave * PROWB));
  auto issue = [&](int stage, int kt) __attribute__((always_inline)) {
    const uint32_t mx = lds_addr(lds) + stage * PHALF + wdst, mw = mx + 2 * PHALF;
    const int64_t off = (int64_t)kt * PROWB;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      dma16(src[2 * i] + off, mx + i * 8 * PROWB);
      dma16(src[2 * i + 1] + off, mw + i * 8 * PROWB);
    }
  };

  // Accumulators start from the bias: block (nb, mb) register r holds
  // C[m][n] with m = m0 + 64wm + 32mb + c and n = n0 + 128wn + 32nb +
  // 8(r/4) + 4hf + r%4, so registers 4q .. 4q+3 take 4 consecutive bias
  // values (one 8-byte load; N is a multiple of 64, so n < N covers all 4).
  // The 16 loads of a lane are issued back to back under one uniform branch
  // (columns past N read a clamped column and take zero), so they cost one
  // memory latency rather than sixteen; the first stage's copies are already
  // in flight.
  issue(0, 0);
  f32x16 acc[4][2];
  {
    u32x2 braw[4][4];
    if (p.bias) {
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int n = n0 + 128 * wn + 32 * nb + 8 * q + 4 * hf;
          braw[nb][q] = *reinterpret_cast<const u32x2*>(p.bias + min(n, p.N - 4));
        }
    } else {
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
#pragma unroll
        for (int q = 0; q < 4; ++q) braw[nb][q] = (u32x2){0u, 0u};
    }
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int n = n0 + 128 * wn + 32 * nb + 8 * q + 4 * hf;
        const T* bt = reinterpret_cast<const T*>(&braw[nb][q]);
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[nb][mb][4 * q + e] = n < p.N ? (float)bt[e] : 0.f;
      }
  }

  // Operand rows 64wm + 32mb + c (x) and 128wn + 32nb + c (W) all have the
  // swizzle sw = (c & 7) ^ ((c >> 3) & 1), so k-step t (chunk 4hf + t, i.e.
  // k = 32hf + 8t .. +7 in both operands) reads at a per-lane base plus
  // stage * 32 KB + 4 KB per block.
  // (32-bit LDS addresses: 8 registers for all eight bases.)
  typedef __attribute__((address_space(3))) const char lchar;
  typedef __attribute__((address_space(3))) const vec8 lvec8;
  const int sw = (c & 7) ^ ((c >> 3) & 1);
  lchar* const lbase = (lchar*)lds;
  lchar* xa[4];
  lchar* wa[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int ch = 16 * ((4 * hf + t) ^ sw);
    xa[t] = lbase + (64 * wm + c) * PROWB + ch;
    wa[t] = lbase + 2 * PHALF + (128 * wn + c) * PROWB + ch;
  }
  // One stage of MFMAs; after the first k-step's MFMAs are issued, `mid`
  // runs (the next stage's copies: their address arithmetic then overlaps
  // the matrix work instead of preceding it).
  auto compute = [&](int stage, auto mid) __attribute__((always_inline)) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      vec8 xo[2], wo[4];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) xo[mb] = *(lvec8*)(xa[t] + stage * PHALF + mb * 32 * PROWB);
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) wo[nb] = *(lvec8*)(wa[t] + stage * PHALF + nb * 32 * PROWB);
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) acc[nb][mb] = H16::mfma(wo[nb], xo[mb], acc[nb][mb]);
      if (t == 0) mid();
    }
  };

  // Two stages: wait for stage kt (own copies), barrier (every wave's copies
  // of kt have landed and every wave is done with kt - 1), compute kt and,
  // inside it, start kt + 1 into kt - 1's buffer.
  const int n_k = p.K / PK;
  for (int kt = 0; kt < n_k; ++kt) {
    wait_vmem<0>();
    barrier_keep_dma();
    compute(kt & 1, [&]() __attribute__((always_inline)) {
      if (kt + 1 < n_k) issue((kt + 1) & 1, kt + 1);
    });
  }

  // Epilogue through LDS (the stage buffers are free once every wave is past
  // its last stage): wave w rounds its 64 x 128 block of C to T and writes it
  // to its own 16 KB, rows of 256 bytes; then each lane reads back whole
  // 16-byte pieces of output rows and stores them, 16 lanes per row of the
  // block (two heads of 128 bytes each: full cache lines).  Row rr keeps
  // 16-byte chunk j at chunk j ^ (rr & 15), and rows 16..31 of each 32 swap
  // the two 8-byte halves of a chunk, so that neither the 8-byte writes (32
  // rows, one column group) nor the 16-byte reads (one row) meet a bank twice.
  __syncthreads();
  char* const ow = lds + wave * (64 * 256);
#pragma unroll
  for (int nb = 0; nb < 4; ++nb)
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int rr = 32 * mb + c, ch = 4 * nb + q;
        const f32x16& a = acc[nb][mb];
        const u32x2 wv = {H16::pack2(a[4 * q], a[4 * q + 1]), H16::pack2(a[4 * q + 2], a[4 * q + 3])};
        *reinterpret_cast<u32x2*>(ow + rr * 256 + ((ch ^ (rr & 15)) << 4) + ((hf ^ (rr >> 4 & 1)) << 3)) = wv;
      }
  __builtin_amdgcn_wave_barrier();
#pragma unroll 4
  for (int i = 0; i < 16; ++i) {
    const int rr = 4 * i + lane / 16, ch = lane % 16;
    u32x4 v = *reinterpret_cast<const u32x4*>(ow + rr * 256 + ((ch ^ (rr & 15)) << 4));
    if (rr >> 4 & 1) v = (u32x4){v[2], v[3], v[0], v[1]};
    const int m = m0 + 64 * wm + rr;
    const int ng = n0 + 128 * wn + 64 * (ch / 8);
    if (m >= p.M || ng >= p.N) continue;
    const int which = ng / p.K;
    const int h = (ng - which * p.K) >> 6;
    const int bb = m / p.S, sq = m - bb * p.S;
    // (selected, not indexed: an indexed kernel-argument array is a memory load)
    T* const ob = which == 0 ? p.out[0] : which == 1 ? p.out[1] : p.out[2];
    T* const orow = ob + (((int64_t)bb * p.H + h) * p.S + sq) * 64;
    __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(orow + 8 * (ch % 8)));  // written once, not read here
  }
}

template <typename T>
int launch_proj(const void* x, const void* w, const void* bias, void* q, void* k, void* v, int B, int S, int H,
                hipStream_t stream) {
  ProjParams<T> p;
  p.x = static_cast<const T*>(x);
  p.w = static_cast<const T*>(w);
  p.bias = static_cast<const T*>(bias);
  p.out[0] = static_cast<T*>(q);
  p.out[1] = static_cast<T*>(k);
  p.out[2] = static_cast<T*>(v);
  p.M = B * S;
  p.K = 64 * H;
  p.N = 3 * p.K;
  p.S = S;
  p.H = H;
  p.tiles_n = (p.N + PN - 1) / PN;
  const int tiles_m = (p.M + PM - 1) / PM;
  p.tiles = tiles_m * p.tiles_n;
  // XCD parts: the cg (dividing the column tiles, 8 / cg dividing the row
  // blocks) with the fewest blocks fetched per round of 32 workgroups.
  p.cg = 0;
  p.prows = p.pcols = 0;
  double best = 0;
  for (int cg = 1; cg <= 8; cg *= 2) {
    if (p.tiles_n % cg || tiles_m % (8 / cg)) continue;
    const int c = p.tiles_n / cg;
    const double cost = (c >= 32 ? 1.0 : 32.0 / c) + (c >= 32 ? 32.0 : c);
    if (!p.cg || cost < best) {
      best = cost;
      p.cg = cg;
      p.pcols = c;
      p.prows = tiles_m / (8 / cg);
    }
  }
  hipLaunchKernelGGL((qkv_proj_kernel<T>), dim3(p.tiles), dim3(PTHREADS), 0, stream, p);
  return hipGetLastError() == hipSuccess ? ATTN_OK : ATTN_E_HIP;
}

}  // namespace

extern "C" int attn_qkv_proj(const void* x, const void* w, const void* bias, void* q, void* k, void* v, int B,
                             int S, int H, int D_h, int dtype, void* stream) {
  if (!x || !w || !q || !k || !v) return ATTN_E_NULL;
  if (B < 1 || S < 1 || H < 1 || D_h != 64) return ATTN_E_SHAPE;
  if (dtype != ATTN_F16 && dtype != ATTN_BF16) return ATTN_E_DTYPE;
  const int64_t M = (int64_t)B * S, d = 64 * (int64_t)H, N = 3 * d;
  if (M > INT32_MAX || N > INT32_MAX) return ATTN_E_SHAPE;
  if (M > INT64_MAX / (2 * d) || N > INT64_MAX / (2 * d)) return ATTN_E_SHAPE;
  const int64_t tiles = ((M + PM - 1) / PM) * ((N + PN - 1) / PN);
  if (tiles > INT32_MAX) return ATTN_E_SHAPE;
  const uintptr_t mis = ((uintptr_t)x | (uintptr_t)w | (uintptr_t)bias | (uintptr_t)q | (uintptr_t)k |
                         (uintptr_t)v) & 15u;
  if (mis) return ATTN_E_ALIGN;
  const uint64_t nx = (uint64_t)M * d * 2, nw = (uint64_t)N * d * 2, nb = bias ? (uint64_t)N * 2 : 0,
                 no = (uint64_t)M * d * 2;  // each of q, k, v: B*H*S*64 elements
  const void* outs[3] = {q, k, v};
  for (int i = 0; i < 3; ++i) {
    if (ranges_overlap(outs[i], no, x, nx) || ranges_overlap(outs[i], no, w, nw) ||
        (bias && ranges_overlap(outs[i], no, bias, nb)))
      return ATTN_E_OVERLAP;
    for (int j = i + 1; j < 3; ++j)
      if (ranges_overlap(outs[i], no, outs[j], no)) return ATTN_E_OVERLAP;
  }
  int n_cu = 0;
  const int dv = check_device(&n_cu);
  if (dv != ATTN_OK) return dv;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (dtype == ATTN_F16) return launch_proj<_Float16>(x, w, bias, q, k, v, B, S, H, s);
  return launch_proj<__bf16>(x, w, bias, q, k, v, B, S, H, s);
}
