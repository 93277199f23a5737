// KV Bridging: the Cross-Decoder's full-attention K and V rows computed from
// the Self-Decoder's hidden states (news page "两天两连更：小米提前亮出V3底牌",
// section "两级KV共享：让模型少跑一半", item KV Bridging), written straight into
// the cache the full layer and its sparse layers read.  One token at the end
// of the cache is the decode-time append.
//
// The operation is a bf16 contraction over the hidden size dm:
//   C[f][m] = sum_k W[f][k] * H[m][k]      (fp32 accumulation, bf16 RNE output)
// with token m = b * n + t and feature f = (kv, g, d) of W [2][Hkv][D][dm];
// C[f][m] goes to cache_kv[b][g][pos0 + t][d].  Both operands are contiguous
// along the reduction, so every MFMA operand is one 16-byte load per lane.
//
// Two kernels:
//  * many tokens (a prefill chunk or a whole prompt): 256 tokens x 256
//    features (two heads' K or V) per work-group of 8 waves, each wave 64
//    tokens x 128 features (two waves per SIMD, so that one's waits and
//    barriers are covered by the other's MFMAs), every feature operand read
//    from LDS serving 4 MFMAs and every token operand 8; the reduction is
//    staged through LDS 32 deep, four stages in flight, by LDS-direct loads
//    issued three stages ahead, and each stage's operands are read into
//    registers while the previous stage's MFMAs run; the work-groups of one
//    token tile sit on one XCD so its
//    L2 serves the tile's hidden rows to all their feature tiles;
//  * a few tokens (decode-time append, up to 64): the weights are the only
//    real traffic, so each work-group takes 16 features x 16 tokens and its 16
//    waves split the reduction, with operands loaded directly from global
//    memory (no reuse to stage) and a fixed-order sum of the 16 partials.

#include "hs2_internal.h"

namespace hs2 {
namespace {

constexpr int kBM = 256;      // tokens per work-group (large kernel)
constexpr int kBN = 256;      // features per work-group: two heads' K or V
constexpr int kBK = 32;       // reduction depth of one LDS stage (64-byte rows)
constexpr int kBStages = 4;   // LDS stages in flight
constexpr int kBWaves = 8;    // waves per work-group (large kernel)
constexpr int kSmallWaves = 16;

__device__ __forceinline__ int xcd_group(int id, int n) {
  // hardware dispatch sends work-group id to XCD id % 8; renumber so that XCD x
  // processes the contiguous range [x * n/8, (x+1) * n/8)
  if (n % 8 != 0) return id;
  return (id & 7) * (n >> 3) + (id >> 3);
}

// Store four features (consecutive d) of token m, already in fp32.
__device__ __forceinline__ void store4(const BridgeArgs& a, int f, int m, f32x4 c) {
  const int b = m / a.n_tok, t = m - b * a.n_tok;
  const int hd = f / kD;                 // (kv, g) of the feature
  const int kv = hd / a.Hkv, g = hd - kv * a.Hkv;
  const int d = f - hd * kD;
  u16* dst = (kv == 0 ? a.k : a.v) +
             ((static_cast<size_t>(b) * a.Hkv + g) * a.kvp + a.pos0 + t) * kD + d;
  const uint2 pk{pack_bf16x2(c[0], c[1]), pack_bf16x2(c[2], c[3])};
  *reinterpret_cast<uint2*>(dst) = pk;
}

// LDS stage layout: 256 rows of 32 bf16 (64 bytes), the 16-byte chunk c of
// row r at slot c ^ ((r >> 1) & 3): a 16-byte operand read is served 128 bytes
// at a time, i.e. 8 lanes = 8 consecutive rows at one chunk, whose rows two
// apart share bank offsets; the swizzle gives those rows distinct slots, so
// the 8 cover all banks once (measured: no bank conflicts; with rows four
// apart separated instead, 20% of the cycles were conflicts).
__device__ __forceinline__ int bslot(int r, int c) { return c ^ ((r >> 1) & 3); }

// grid: Hkv * ceil(M / 256) work-groups of 512 threads.
__global__ __launch_bounds__(kBWaves * 64, 1) void bridge_gemm_kernel(BridgeArgs a) {
  __shared__ __align__(16) u16 wl[kBStages][kBN * kBK];
  __shared__ __align__(16) u16 hl[kBStages][kBM * kBK];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int col = lane & 15, grp = lane >> 4;
  const int n_ft = a.Hkv;                      // 2 Hkv D / 256
  const int lin = xcd_group(blockIdx.x, gridDim.x);
  const int ft = lin % n_ft;
  const int m0 = (lin / n_ft) * kBM;
  const int f0 = ft * kBN;
  const int wm = wave & 3, wn = wave >> 2;     // the wave's 64 tokens and 128 features

  // One stage: 16 LDS-direct loads of 1 KB (16 rows each) per operand, 2 per
  // wave and operand: lane l fills slot l & 3 of row 16 i + (l >> 2) with that
  // row's chunk (l & 3) ^ swizzle.  Hidden rows past M repeat the last.  Each
  // load is a scalar base (the work-group's first row at the stage's column)
  // plus a fixed per-lane byte offset, its LDS address a scalar in m0.  Issued
  // from inline assembly, so that the compiler, which cannot tell the stage
  // buffers apart, does not wait for them before every LDS read; the waits
  // are explicit (vector memory operations complete in order).
  uint32_t w_off[2], h_off[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int r = 32 * wave + 16 * u + (lane >> 2);
    const int c = bslot(r, lane & 3);         // chunk for slot lane & 3 (an involution)
    w_off[u] = static_cast<uint32_t>((static_cast<size_t>(r) * a.dm + 8 * c) * 2);
    const int m = min(m0 + r, a.M - 1);
    h_off[u] = static_cast<uint32_t>((static_cast<size_t>(m - m0) * a.dm + 8 * c) * 2);
  }
  const u16* w_base = a.w + static_cast<size_t>(f0) * a.dm;
  const u16* h_base = a.hidden + static_cast<size_t>(m0) * a.dm;
  const uint32_t wl0 = __builtin_amdgcn_readfirstlane(
      static_cast<uint32_t>(reinterpret_cast<uintptr_t>(&wl[0][32 * wave * kBK])));
  const uint32_t hl0 = __builtin_amdgcn_readfirstlane(
      static_cast<uint32_t>(reinterpret_cast<uintptr_t>(&hl[0][32 * wave * kBK])));
  constexpr uint32_t kStageBytes = kBN * kBK * 2;
  // load number i (0..3) of stage kt: rows 16 (i >> 1) .. of this wave's 32,
  // of the weights (i even) or the hidden states (i odd)
  auto dma_one = [&](int kt, int i) {
    const uint32_t sb = (kt % kBStages) * kStageBytes + 16 * (i >> 1) * kBK * 2;
    if (i & 1)
      asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
                   :: "s"(hl0 + sb), "v"(h_off[i >> 1]), "s"(h_base + kt * kBK) : "memory", "m0");
    else
      asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
                   :: "s"(wl0 + sb), "v"(w_off[i >> 1]), "s"(w_base + kt * kBK) : "memory", "m0");
  };
  auto dma_stage = [&](int kt) {
#pragma unroll
    for (int i = 0; i < 4; ++i) dma_one(kt, i);
  };
  // the wave's operands of one stage: 8 feature blocks and 4 token blocks
  auto read_ops = [&](int kt, bf16x8 (&wa)[8], bf16x8 (&hb)[4]) {
    const int buf = kt % kBStages;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int rw = 128 * wn + 16 * i + col;
      wa[i] = as_bf16x8(*reinterpret_cast<const u32x4*>(&wl[buf][rw * kBK + 8 * bslot(rw, grp)]));
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int rh = 64 * wm + 16 * j + col;
      hb[j] = as_bf16x8(*reinterpret_cast<const u32x4*>(&hl[buf][rh * kBK + 8 * bslot(rh, grp)]));
    }
  };

  f32x4 acc[8][4];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Stage kt + 3 is loaded at the start of stage kt (into the buffer of stage
  // kt - 1, whose operands were read during stage kt - 2); stage kt + 1 must
  // be in LDS by the end of stage kt - 1, since its operands are read while
  // stage kt's MFMAs run (two register sets).
  const int nk = a.dm / kBK;
  dma_stage(0);
  if (nk > 1) dma_stage(1);
  if (nk > 2) dma_stage(2);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  bf16x8 wa[2][8], hb[2][4];
  read_ops(0, wa[0], hb[0]);
  for (int kt = 0; kt < nk; kt += 2) {
    // two stages per trip (nk is even), so that the register sets are named
    // statically
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int s = kt + h;
      const bool more = s + 3 < nk;
      if (more) dma_stage(s + 3);
      read_ops(min(s + 1, nk - 1), wa[h ^ 1], hb[h ^ 1]);
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = mfma_16x16x32(wa[h][i], hb[h][j], acc[i][j]);
      // stage s + 2 (read during stage s + 1): only stage s + 3's 4 loads,
      // if issued, are newer
      if (more) asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
      else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  // C[feature 4 grp + e][token col] of block (i, j)
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int m = m0 + 64 * wm + 16 * j + col;
    if (m >= a.M) continue;
#pragma unroll
    for (int i = 0; i < 8; ++i) store4(a, f0 + 128 * wn + 16 * i + 4 * grp, m, acc[i][j]);
  }
}

// grid: (2 Hkv D / 16, ceil(M / 16)) work-groups of 16 waves.
__global__ __launch_bounds__(kSmallWaves * 64) void bridge_small_kernel(BridgeArgs a) {
  __shared__ f32x4 red[kSmallWaves][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 15, grp = lane >> 4;
  const int f = 16 * blockIdx.x + col;                    // A row: a feature
  const int m = min(16 * static_cast<int>(blockIdx.y) + col, a.M - 1);   // B column: a token
  const u16* wp = a.w + static_cast<size_t>(f) * a.dm + 8 * grp;
  const u16* hp = a.hidden + static_cast<size_t>(m) * a.dm + 8 * grp;
  const int nks = a.dm / 32;
  f32x4 acc{0.f, 0.f, 0.f, 0.f};
  // wave w takes reduction steps w, w + 16, ...; eight loads of each operand in
  // flight per round (one round at d_model = 4096)
  constexpr int kU = 8;
  for (int s0 = wave; s0 < nks; s0 += kU * kSmallWaves) {
    u32x4 wv[kU], hv[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int s = s0 + u * kSmallWaves;
      if (s < nks) {
        wv[u] = load_u32x4(wp + 32 * s);
        hv[u] = load_u32x4(hp + 32 * s);
      }
    }
#pragma unroll
    for (int u = 0; u < kU; ++u)
      if (s0 + u * kSmallWaves < nks) acc = mfma_16x16x32(as_bf16x8(wv[u]), as_bf16x8(hv[u]), acc);
  }
  red[wave][lane] = acc;
  __syncthreads();
  if (wave != 0) return;
  f32x4 c = red[0][lane];
  for (int w = 1; w < kSmallWaves; ++w) c += red[w][lane];
  const int mo = 16 * blockIdx.y + col;
  if (mo < a.M) store4(a, 16 * blockIdx.x + 4 * grp, mo, c);
}

}  // namespace

hipError_t launch_kv_bridge(const BridgeArgs& a, hipStream_t st) {
  if (a.M <= 64) {
    dim3 grid(2 * a.Hkv * kD / 16, (a.M + 15) / 16);
    hipLaunchKernelGGL(bridge_small_kernel, grid, dim3(kSmallWaves * 64), 0, st, a);
  } else {
    const int n_wg = a.Hkv * ((a.M + kBM - 1) / kBM);
    hipLaunchKernelGGL(bridge_gemm_kernel, dim3(n_wg), dim3(kBWaves * 64), 0, st, a);
  }
  return hipGetLastError();
}

}  // namespace hs2
