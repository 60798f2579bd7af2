// Gated DeltaNet decode block for gfx950: HIP kernels and the C ABI of include/gdn_block.h.
//
// One decode call is three launches on the caller's stream:
//   norm_kernel   one workgroup per row: h = bf16(x + residual), residual <- h,
//                 xn = bf16(h * rstd * (1 + w)) into scratch ("sgl-amd-mono PR #89",
//                 Kernels before and after: the fused residual add + Gemma norm).
//   gemv_kernel   in_proj_qkvz and in_proj_ba as one skinny GEMM on the bf16 MFMA
//                 (v_mfma_f32_16x16x32_bf16: 16 weight rows x 16 decode rows per tile).
//                 K is split over workgroups; the last workgroup of a tile to finish
//                 (an atomic counter, no waiting) adds the partials in split order, rounds
//                 to bf16 and runs the tile's epilogue: the causal conv update + SiLU for
//                 q|k|v channels (rolling the conv state in place), or storing z / b / a.
//   gdn_kernel    one workgroup per (value head, row): L2 norms, gates, the gated delta
//                 rule on the head's dk x dv state held in registers, the state store,
//                 and the gated RMSNorm into the core output.
//
// Every reduction runs in a fixed order that does not depend on the row count, so a
// row's results do not change with the other rows (batch invariance, "sgl-amd-mono PR
// #89", Kernel checks).
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <string>

#include "gdn_block.h"

namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(4))) unsigned u32x4_t;

constexpr int kConvW = 4;      // conv width; create() refuses any other
constexpr int kThreads = 256;  // every kernel runs 4 waves of 64

// ---------------------------------------------------------------------------------------
// scalar helpers

__device__ __forceinline__ float bf2f(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// round-to-nearest-even f32 -> bf16 (inputs are finite)
__device__ __forceinline__ uint16_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ float silu(float x) { return x / (1.0f + expf(-x)); }

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// sum over the 256 threads of a workgroup in a fixed order; `lds` holds 4 floats
__device__ __forceinline__ float block_sum(float v, float* lds) {
  v = wave_sum(v);
  if ((threadIdx.x & 63) == 0) lds[threadIdx.x >> 6] = v;
  __syncthreads();
  const float r = (lds[0] + lds[1]) + (lds[2] + lds[3]);
  __syncthreads();
  return r;
}

// cross-workgroup hand-off: coherent single accesses plus a wait for this wave's stores
__device__ __forceinline__ void store_agent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_agent(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void wait_stores() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t v) { return __builtin_bit_cast(bf16x8_t, v); }

__device__ __forceinline__ uint32_t pack2(uint16_t lo, uint16_t hi) { return (uint32_t)lo | ((uint32_t)hi << 16); }

// ---------------------------------------------------------------------------------------
// 1. residual add + Gemma RMSNorm, one workgroup per row

constexpr int kNormMaxChunks = 8;  // 16-byte chunks per thread: H <= 8 * 8 * 256

template <bool HAS_RES>
__global__ __launch_bounds__(kThreads) void norm_kernel(const uint16_t* __restrict__ x,
                                                        uint16_t* __restrict__ residual,
                                                        const uint16_t* __restrict__ w,
                                                        uint16_t* __restrict__ xn, int H, float eps) {
  __shared__ float red[4];
  const int row = blockIdx.x;
  const int nchunk = H >> 3;
  const uint4* xp = reinterpret_cast<const uint4*>(x + (size_t)row * H);
  uint4* rp = reinterpret_cast<uint4*>(residual + (size_t)row * H);
  uint4 hv[kNormMaxChunks];
  float ss = 0.0f;
#pragma unroll
  for (int c = 0; c < kNormMaxChunks; ++c) {
    const int idx = threadIdx.x + c * kThreads;
    if (idx < nchunk) {
      uint4 a = xp[idx];
      if (HAS_RES) {
        const uint4 b = rp[idx];
        uint32_t* pa = reinterpret_cast<uint32_t*>(&a);
        const uint32_t* pb = reinterpret_cast<const uint32_t*>(&b);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint16_t lo = f2bf(bf2f((uint16_t)pa[q]) + bf2f((uint16_t)pb[q]));
          const uint16_t hi = f2bf(bf2f((uint16_t)(pa[q] >> 16)) + bf2f((uint16_t)(pb[q] >> 16)));
          pa[q] = pack2(lo, hi);
        }
      }
      hv[c] = a;
      const uint32_t* ph = reinterpret_cast<const uint32_t*>(&a);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float l = bf2f((uint16_t)ph[q]), h = bf2f((uint16_t)(ph[q] >> 16));
        ss = fmaf(l, l, ss);
        ss = fmaf(h, h, ss);
      }
    }
  }
  ss = block_sum(ss, red);
  const float rstd = 1.0f / sqrtf(ss / (float)H + eps);
  const uint4* wp = reinterpret_cast<const uint4*>(w);
  uint4* op = reinterpret_cast<uint4*>(xn + (size_t)row * H);
#pragma unroll
  for (int c = 0; c < kNormMaxChunks; ++c) {
    const int idx = threadIdx.x + c * kThreads;
    if (idx < nchunk) {
      rp[idx] = hv[c];  // each thread rewrites only the residual chunks it read itself
      const uint4 wv = wp[idx];
      const uint32_t* ph = reinterpret_cast<const uint32_t*>(&hv[c]);
      const uint32_t* pw = reinterpret_cast<const uint32_t*>(&wv);
      uint4 o;
      uint32_t* po = reinterpret_cast<uint32_t*>(&o);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint16_t lo = f2bf(bf2f((uint16_t)ph[q]) * rstd * (1.0f + bf2f((uint16_t)pw[q])));
        const uint16_t hi =
            f2bf(bf2f((uint16_t)(ph[q] >> 16)) * rstd * (1.0f + bf2f((uint16_t)(pw[q] >> 16))));
        po[q] = pack2(lo, hi);
      }
      op[idx] = o;
    }
  }
}

// ---------------------------------------------------------------------------------------
// 2. projections on the MFMA, split-K with a last-arriver reduction, conv epilogue

struct GemvArgs {
  const uint16_t* xn;      // [R, H]
  const uint16_t* wq;      // in_proj_qkvz [Nq, H]
  const uint16_t* wb;      // in_proj_ba [Nb, H]
  const int32_t* idx;      // [R]
  const uint16_t* conv_w;  // [Cd, 4]
  uint16_t* conv_state;    // [slots, 3, Cd]
  uint16_t* cbuf;          // [R, Cd]   conv outputs (bf16, after SiLU)
  uint16_t* zbuf;          // [R, nv*dv]
  uint16_t* babuf;         // [R, 2*nv] b then a
  float* part;             // [S, T, 256] split partials
  unsigned* cnt;           // [T] arrivals per tile, reset by the last arriver
  int H, R, Tq, T, Nq, Nb;
  int nk, dk, nv, dv, r, GW, Cd, slots;
};

__device__ __forceinline__ void gemv_epilogue(const GemvArgs& a, bool isq, int ch, int n, float v, int N) {
  if (n >= a.R || ch >= N) return;
  const uint16_t yb = f2bf(v);
  if (isq) {
    const int g = ch / a.GW, o = ch - g * a.GW;
    const int two_dk = 2 * a.dk, rdv = a.r * a.dv;
    if (o < two_dk + rdv) {
      int cc;
      if (o < a.dk)
        cc = g * a.dk + o;
      else if (o < two_dk)
        cc = a.nk * a.dk + g * a.dk + (o - a.dk);
      else
        cc = 2 * a.nk * a.dk + g * rdv + (o - two_dk);
      const int slot = a.idx[n];
      if (slot <= 0 || slot >= a.slots) return;  // pad row: no conv state write
      uint16_t* st = a.conv_state + (size_t)slot * (kConvW - 1) * a.Cd + cc;
      const uint16_t* wc = a.conv_w + (size_t)cc * kConvW;
      uint16_t prev[kConvW - 1];
      float acc = 0.0f;
#pragma unroll
      for (int j = 0; j < kConvW - 1; ++j) {
        prev[j] = st[(size_t)j * a.Cd];
        acc = fmaf(bf2f(wc[j]), bf2f(prev[j]), acc);
      }
      acc = fmaf(bf2f(wc[kConvW - 1]), bf2f(yb), acc);
#pragma unroll
      for (int j = 0; j < kConvW - 2; ++j) st[(size_t)j * a.Cd] = prev[j + 1];
      st[(size_t)(kConvW - 2) * a.Cd] = yb;
      a.cbuf[(size_t)n * a.Cd + cc] = f2bf(silu(acc));
    } else {
      a.zbuf[(size_t)n * a.nv * a.dv + g * rdv + (o - two_dk - rdv)] = yb;
    }
  } else {
    const int g = ch / (2 * a.r), o = ch - g * 2 * a.r;
    const int dst = (o < a.r) ? (g * a.r + o) : (a.nv + g * a.r + (o - a.r));
    a.babuf[(size_t)n * 2 * a.nv + dst] = yb;
  }
}

// grid: (T tiles of 16 output channels, S splits of K); 4 waves each take a quarter of the
// workgroup's K range. Lane l of a wave: A operand = weight row (l % 16) of the tile,
// B operand = decode row (l % 16), both at k offset 8 * (l / 16) of each 32-wide step.
template <int U>
__global__ __launch_bounds__(kThreads) void gemv_kernel(GemvArgs a) {
  __shared__ float red[4][256];
  __shared__ int is_last;
  const int t = blockIdx.x, s = blockIdx.y, S = gridDim.y;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const bool isq = t < a.Tq;
  const uint16_t* W = isq ? a.wq : a.wb;
  const int N = isq ? a.Nq : a.Nb;
  const int row0 = (isq ? t : t - a.Tq) * 16;
  const int q16 = lane & 15, kg = lane >> 4;
  // rows past the end of the matrix or past the decode rows are clamped to valid memory;
  // their MFMA outputs land in tile positions the epilogue never stores
  const int wrow = min(row0 + q16, N - 1);
  const int xrow = min(q16, a.R - 1);
  const int Kw = a.H / (S * 4);
  const int k0 = (s * 4 + wave) * Kw + 8 * kg;
  const u32x4_t* wp = reinterpret_cast<const u32x4_t*>(W + (size_t)wrow * a.H + k0);
  const u32x4_t* xp = reinterpret_cast<const u32x4_t*>(a.xn + (size_t)xrow * a.H + k0);
  f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
  const int steps = Kw >> 5;
  for (int st = 0; st < steps; st += U) {
    u32x4_t wv[U], xv[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      wv[u] = __builtin_nontemporal_load(wp + (st + u) * 4);
      xv[u] = xp[(st + u) * 4];
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(wv[u]), as_bf16x8(xv[u]), acc, 0, 0, 0);
  }
  // D layout: lane l holds channels 4 * (l / 16) + i (i = 0..3) of decode row l % 16
#pragma unroll
  for (int i = 0; i < 4; ++i) red[wave][i * 64 + lane] = acc[i];
  __syncthreads();
  const int tid = threadIdx.x;
  const int en = tid >> 4, em = tid & 15;  // this thread's (decode row, channel) of the tile
  const int src = (em & 3) * 64 + (em >> 2) * 16 + en;
  float v = ((red[0][src] + red[1][src]) + red[2][src]) + red[3][src];
  if (S > 1) {
    // Hand the partial to the tile's last workgroup. Partials travel as agent-scope
    // atomic stores and loads, which are coherent across the XCDs' L2s one access at a
    // time; the wait below makes them complete before this workgroup's arrival is
    // counted. (A device-wide fence here would write back and invalidate a whole L2 in
    // every workgroup.)
    store_agent(&a.part[((size_t)s * a.T + t) * 256 + tid], v);
    wait_stores();
    __syncthreads();
    if (tid == 0)
      is_last = __hip_atomic_fetch_add(&a.cnt[t], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                (unsigned)(S - 1);
    __syncthreads();
    if (!is_last) return;
    v = 0.0f;
    for (int q = 0; q < S; ++q) v += load_agent(&a.part[((size_t)q * a.T + t) * 256 + tid]);
    if (tid == 0) __hip_atomic_store(&a.cnt[t], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  gemv_epilogue(a, isq, row0 + em, en, v, N);
}

// ---------------------------------------------------------------------------------------
// 3. L2 norms, gates, gated delta rule, gated RMSNorm; one workgroup per (value head, row)

struct GdnArgs {
  const int32_t* idx;       // [R]
  const uint16_t* cbuf;     // [R, Cd]
  const uint16_t* zbuf;     // [R, nv*dv]
  const uint16_t* babuf;    // [R, 2*nv]
  const float* A_log;       // [nv]
  const uint16_t* dt_bias;  // [nv]
  const uint16_t* gnw;      // [dv]
  void* ssm;                // [slots, nv, dk, dv]
  uint16_t* core;           // [R, nv*dv]
  int nk, nv, r, Cd, slots;
  float l2eps, geps;
};

template <typename ST>
struct StateIO;

template <>
struct StateIO<float> {
  static __device__ __forceinline__ void load(const void* base, size_t off, float* v) {
    const float4 q = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(base) + off);
    v[0] = q.x, v[1] = q.y, v[2] = q.z, v[3] = q.w;
  }
  static __device__ __forceinline__ void store(void* base, size_t off, const float* v) {
    *reinterpret_cast<float4*>(reinterpret_cast<float*>(base) + off) = make_float4(v[0], v[1], v[2], v[3]);
  }
};

template <>
struct StateIO<uint16_t> {
  static __device__ __forceinline__ void load(const void* base, size_t off, float* v) {
    const uint2 q = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint16_t*>(base) + off);
    v[0] = bf2f((uint16_t)q.x), v[1] = bf2f((uint16_t)(q.x >> 16));
    v[2] = bf2f((uint16_t)q.y), v[3] = bf2f((uint16_t)(q.y >> 16));
  }
  static __device__ __forceinline__ void store(void* base, size_t off, const float* v) {
    uint2 q;
    q.x = pack2(f2bf(v[0]), f2bf(v[1]));
    q.y = pack2(f2bf(v[2]), f2bf(v[3]));
    *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(base) + off) = q;
  }
};

template <int DK, int DV, typename ST>
__global__ __launch_bounds__(kThreads) void gdn_kernel(GdnArgs a) {
  constexpr int NCQ = DV / 4;          // column quads
  constexpr int NRG = kThreads / NCQ;  // row groups
  constexpr int RPT = DK / NRG;        // state rows per thread
  static_assert(NRG * NCQ == kThreads && RPT * NRG == DK, "tile shape");
  __shared__ float qs[DK], ks[DK];
  __shared__ float red[NRG][DV];
  __shared__ float vec[DV];
  __shared__ float scal[4];
  __shared__ float bsum[4];

  const int h = blockIdx.x, n = blockIdx.y, tid = threadIdx.x;
  const int slot = a.idx[n];
  uint16_t* core = a.core + (size_t)n * a.nv * DV + (size_t)h * DV;
  if (slot <= 0 || slot >= a.slots) {  // pad row: a zero core row, no state touched
    for (int j = tid; j < DV; j += kThreads) core[j] = 0;
    return;
  }
  const int kap = h / a.r;
  const int cq = tid % NCQ, rg = tid / NCQ;
  const size_t sbase = (((size_t)slot * a.nv + h) * DK) * DV + 4 * cq;

  float S[RPT][4];
#pragma unroll
  for (int m = 0; m < RPT; ++m) StateIO<ST>::load(a.ssm, sbase + (size_t)(rg + NRG * m) * DV, S[m]);

  const uint16_t* crow = a.cbuf + (size_t)n * a.Cd;
  for (int i = tid; i < DK; i += kThreads) {
    qs[i] = bf2f(crow[kap * DK + i]);
    ks[i] = bf2f(crow[a.nk * DK + kap * DK + i]);
  }
  __syncthreads();
  if (tid < 64) {
    float sq = 0.0f;
    for (int i = tid; i < DK; i += 64) sq = fmaf(qs[i], qs[i], sq);
    sq = wave_sum(sq);
    if (tid == 0) scal[0] = sq;
  } else if (tid < 128) {
    float sk = 0.0f;
    for (int i = tid - 64; i < DK; i += 64) sk = fmaf(ks[i], ks[i], sk);
    sk = wave_sum(sk);
    if (tid == 64) scal[1] = sk;
  } else if (tid == 128) {
    const uint16_t* ba = a.babuf + (size_t)n * 2 * a.nv;
    const float b = bf2f(ba[h]);
    const float x = bf2f(ba[a.nv + h]) + bf2f(a.dt_bias[h]);
    const float sp = x > 20.0f ? x : log1pf(expf(x));
    scal[2] = expf(-expf(a.A_log[h]) * sp);  // exp(g)
    scal[3] = 1.0f / (1.0f + expf(-b));       // beta
  }
  __syncthreads();
  const float qscale = (1.0f / sqrtf(scal[0] + a.l2eps)) * (1.0f / sqrtf((float)DK));
  const float kscale = 1.0f / sqrtf(scal[1] + a.l2eps);
  const float decay = scal[2], beta = scal[3];

  float part[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int m = 0; m < RPT; ++m) {
    const float kh = ks[rg + NRG * m] * kscale;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      S[m][c] *= decay;
      part[c] = fmaf(S[m][c], kh, part[c]);
    }
  }
#pragma unroll
  for (int c = 0; c < 4; ++c) red[rg][4 * cq + c] = part[c];
  __syncthreads();
  if (tid < DV) {
    float u = 0.0f;
#pragma unroll
    for (int q = 0; q < NRG; ++q) u += red[q][tid];
    const float v = bf2f(crow[2 * a.nk * DK + h * DV + tid]);
    vec[tid] = beta * (v - u);
  }
  __syncthreads();
  float d[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) d[c] = vec[4 * cq + c], part[c] = 0.0f;
#pragma unroll
  for (int m = 0; m < RPT; ++m) {
    const int i = rg + NRG * m;
    const float kh = ks[i] * kscale, qh = qs[i] * qscale;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      S[m][c] = fmaf(kh, d[c], S[m][c]);
      part[c] = fmaf(S[m][c], qh, part[c]);
    }
    StateIO<ST>::store(a.ssm, sbase + (size_t)i * DV, S[m]);
  }
#pragma unroll
  for (int c = 0; c < 4; ++c) red[rg][4 * cq + c] = part[c];
  __syncthreads();
  float ob = 0.0f;
  if (tid < DV) {
    float o = 0.0f;
#pragma unroll
    for (int q = 0; q < NRG; ++q) o += red[q][tid];
    ob = bf2f(f2bf(o));
  }
  const float ss = block_sum(tid < DV ? ob * ob : 0.0f, bsum);
  const float rstd = 1.0f / sqrtf(ss / (float)DV + a.geps);
  if (tid < DV) {
    const float z = bf2f(a.zbuf[(size_t)n * a.nv * DV + (size_t)h * DV + tid]);
    core[tid] = f2bf(ob * rstd * bf2f(a.gnw[tid]) * silu(z));
  }
}

}  // namespace

// =======================================================================================
// host side: the C ABI

struct gdn_block {
  gdn_block_config cfg;
  int device;
  int nq, nb, cd, tq, t, splits, unroll;
  void* scratch;
  uint16_t* xn;
  float* part;
  unsigned* cnt;
  uint16_t* cbuf;
  uint16_t* zbuf;
  uint16_t* babuf;
  std::string err;
};

namespace {

thread_local std::string g_create_error;

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

std::string check_config(const gdn_block_config* c) {
  std::string why;
  auto add = [&](const std::string& s) { why += (why.empty() ? "" : "; ") + s; };
  if (c->hidden <= 0 || c->hidden % 256 != 0 || c->hidden > 16384)
    add("hidden must be a positive multiple of 256 up to 16384 (got " + std::to_string(c->hidden) + ")");
  if (c->num_k_heads <= 0 || c->num_v_heads <= 0 || c->num_v_heads % c->num_k_heads != 0)
    add("num_v_heads must be a positive multiple of num_k_heads");
  if (!(c->head_k_dim == 32 || c->head_k_dim == 64 || c->head_k_dim == 128))
    add("head_k_dim must be 32, 64 or 128");
  if (c->head_v_dim != c->head_k_dim) add("head_v_dim must equal head_k_dim");
  if (c->conv_width != kConvW) add("conv_width must be 4");
  if (c->num_state_slots < 2) add("num_state_slots must be at least 2 (slot 0 is the pad slot)");
  if (c->max_rows < 1 || c->max_rows > GDN_MAX_ROWS) add("max_rows must be in 1..16");
  if (c->qkvz_format != GDN_FMT_BF16 && c->qkvz_format != GDN_FMT_MXFP4)
    add("qkvz_format must be GDN_FMT_BF16 or GDN_FMT_MXFP4");
  if (c->qkvz_format == GDN_FMT_MXFP4) add("MXFP4 in_proj_qkvz is not available in this build");
  if (c->ssm_state_dtype != GDN_STATE_F32 && c->ssm_state_dtype != GDN_STATE_BF16)
    add("ssm_state_dtype must be GDN_STATE_F32 or GDN_STATE_BF16");
  if (c->has_residual != 0 && c->has_residual != 1) add("has_residual must be 0 or 1");
  auto bad_eps = [](float e) { return !(e > 0.0f) || !std::isfinite(e); };
  if (bad_eps(c->norm_eps) || bad_eps(c->gated_norm_eps) || bad_eps(c->l2norm_eps))
    add("every eps must be positive and finite");
  return why;
}

int fail(gdn_block* b, int code, const std::string& msg) {
  b->err = msg;
  return code;
}

template <int U>
void launch_gemv(const gdn_block* b, const GemvArgs& ga, hipStream_t st) {
  hipLaunchKernelGGL(gemv_kernel<U>, dim3(b->t, b->splits), dim3(kThreads), 0, st, ga);
}

template <int D>
void launch_gdn_d(const gdn_block* b, const GdnArgs& ga, int rows, hipStream_t st) {
  if (b->cfg.ssm_state_dtype == GDN_STATE_F32)
    hipLaunchKernelGGL((gdn_kernel<D, D, float>), dim3(b->cfg.num_v_heads, rows), dim3(kThreads), 0, st, ga);
  else
    hipLaunchKernelGGL((gdn_kernel<D, D, uint16_t>), dim3(b->cfg.num_v_heads, rows), dim3(kThreads), 0, st, ga);
}

}  // namespace

extern "C" int gdn_block_create(const gdn_block_config* cfg, gdn_block_t* out) {
  if (out) *out = nullptr;
  if (!cfg || !out) {
    g_create_error = "gdn_block_create: cfg and out must not be NULL";
    return GDN_E_INVALID_ARG;
  }
  const std::string why = check_config(cfg);
  if (!why.empty()) {
    g_create_error = "gdn_block_create: unsupported configuration: " + why;
    return GDN_E_UNSUPPORTED;
  }
  gdn_block* b = new gdn_block();
  b->cfg = *cfg;
  const int H = cfg->hidden, nk = cfg->num_k_heads, dk = cfg->head_k_dim, nv = cfg->num_v_heads,
            dv = cfg->head_v_dim;
  b->nq = 2 * nk * dk + 2 * nv * dv;
  b->nb = 2 * nv;
  b->cd = 2 * nk * dk + nv * dv;
  b->tq = b->nq / 16;
  b->t = b->tq + (b->nb + 15) / 16;
  // K splits: enough workgroups to cover the chip twice, each wave keeping whole 32-wide
  // steps; the count depends on the shape only, never on the row count
  int S = 1;
  while (S < 8 && b->t * S < 512 && H % (4 * 2 * S * 32) == 0) S *= 2;
  b->splits = S;
  const int steps = H / (4 * S * 32);
  b->unroll = steps % 8 == 0 ? 8 : steps % 4 == 0 ? 4 : steps % 2 == 0 ? 2 : 1;

  const int R = cfg->max_rows;
  size_t off = 0;
  const size_t o_xn = off;
  off = align_up(off + (size_t)R * H * 2, 256);
  const size_t o_part = off;
  off = align_up(off + (S > 1 ? (size_t)S * b->t * 256 * 4 : 0), 256);
  const size_t o_cnt = off;
  off = align_up(off + (size_t)b->t * 4, 256);
  const size_t o_c = off;
  off = align_up(off + (size_t)R * b->cd * 2, 256);
  const size_t o_z = off;
  off = align_up(off + (size_t)R * nv * dv * 2, 256);
  const size_t o_ba = off;
  off = align_up(off + (size_t)R * 2 * nv * 2, 256);

  hipError_t e = hipGetDevice(&b->device);
  if (e == hipSuccess) e = hipMalloc(&b->scratch, off);
  if (e == hipSuccess) e = hipMemset(static_cast<char*>(b->scratch) + o_cnt, 0, (size_t)b->t * 4);
  if (e == hipSuccess) e = hipDeviceSynchronize();
  if (e != hipSuccess) {
    g_create_error = std::string("gdn_block_create: HIP error: ") + hipGetErrorString(e);
    if (b->scratch) (void)hipFree(b->scratch);
    delete b;
    return GDN_E_HIP;
  }
  char* base = static_cast<char*>(b->scratch);
  b->xn = reinterpret_cast<uint16_t*>(base + o_xn);
  b->part = reinterpret_cast<float*>(base + o_part);
  b->cnt = reinterpret_cast<unsigned*>(base + o_cnt);
  b->cbuf = reinterpret_cast<uint16_t*>(base + o_c);
  b->zbuf = reinterpret_cast<uint16_t*>(base + o_z);
  b->babuf = reinterpret_cast<uint16_t*>(base + o_ba);
  g_create_error.clear();
  *out = b;
  return GDN_OK;
}

extern "C" int gdn_block_decode(gdn_block_t b, const void* x, void* residual, const gdn_block_weights* w,
                                void* conv_state, void* ssm_state, const int32_t* state_idx, int32_t rows,
                                void* core_out, void* stream) {
  if (!b) return GDN_E_INVALID_ARG;
  const gdn_block_config& c = b->cfg;
  if (rows < 0 || rows > c.max_rows)
    return fail(b, GDN_E_INVALID_ARG,
                "gdn_block_decode: rows must be in 0.." + std::to_string(c.max_rows) + " (got " +
                    std::to_string(rows) + ")");
  if (!w) return fail(b, GDN_E_INVALID_ARG, "gdn_block_decode: weights must not be NULL");
  const void* ptrs[] = {x, residual, conv_state, ssm_state, state_idx, core_out, w->norm_w, w->w_qkvz,
                        w->w_ba, w->conv_w, w->A_log, w->dt_bias, w->gated_norm_w};
  const char* names[] = {"x", "residual", "conv_state", "ssm_state", "state_idx", "core_out", "norm_w",
                         "w_qkvz", "w_ba", "conv_w", "A_log", "dt_bias", "gated_norm_w"};
  for (size_t i = 0; i < sizeof(ptrs) / sizeof(ptrs[0]); ++i) {
    if (!ptrs[i]) return fail(b, GDN_E_INVALID_ARG, std::string("gdn_block_decode: ") + names[i] + " is NULL");
    if (!aligned16(ptrs[i]))
      return fail(b, GDN_E_INVALID_ARG, std::string("gdn_block_decode: ") + names[i] + " is not 16-byte aligned");
  }
  if (rows == 0) return GDN_OK;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int H = c.hidden;

  if (c.has_residual)
    hipLaunchKernelGGL(norm_kernel<true>, dim3(rows), dim3(kThreads), 0, st, static_cast<const uint16_t*>(x),
                       static_cast<uint16_t*>(residual), static_cast<const uint16_t*>(w->norm_w), b->xn, H,
                       c.norm_eps);
  else
    hipLaunchKernelGGL(norm_kernel<false>, dim3(rows), dim3(kThreads), 0, st, static_cast<const uint16_t*>(x),
                       static_cast<uint16_t*>(residual), static_cast<const uint16_t*>(w->norm_w), b->xn, H,
                       c.norm_eps);

  GemvArgs ga;
  ga.xn = b->xn;
  ga.wq = static_cast<const uint16_t*>(w->w_qkvz);
  ga.wb = static_cast<const uint16_t*>(w->w_ba);
  ga.idx = state_idx;
  ga.conv_w = static_cast<const uint16_t*>(w->conv_w);
  ga.conv_state = static_cast<uint16_t*>(conv_state);
  ga.cbuf = b->cbuf;
  ga.zbuf = b->zbuf;
  ga.babuf = b->babuf;
  ga.part = b->part;
  ga.cnt = b->cnt;
  ga.H = H;
  ga.R = rows;
  ga.Tq = b->tq;
  ga.T = b->t;
  ga.Nq = b->nq;
  ga.Nb = b->nb;
  ga.nk = c.num_k_heads;
  ga.dk = c.head_k_dim;
  ga.nv = c.num_v_heads;
  ga.dv = c.head_v_dim;
  ga.r = c.num_v_heads / c.num_k_heads;
  ga.GW = 2 * c.head_k_dim + 2 * ga.r * c.head_v_dim;
  ga.Cd = b->cd;
  ga.slots = c.num_state_slots;
  switch (b->unroll) {
    case 8: launch_gemv<8>(b, ga, st); break;
    case 4: launch_gemv<4>(b, ga, st); break;
    case 2: launch_gemv<2>(b, ga, st); break;
    default: launch_gemv<1>(b, ga, st); break;
  }

  GdnArgs da;
  da.idx = state_idx;
  da.cbuf = b->cbuf;
  da.zbuf = b->zbuf;
  da.babuf = b->babuf;
  da.A_log = w->A_log;
  da.dt_bias = static_cast<const uint16_t*>(w->dt_bias);
  da.gnw = static_cast<const uint16_t*>(w->gated_norm_w);
  da.ssm = ssm_state;
  da.core = static_cast<uint16_t*>(core_out);
  da.nk = c.num_k_heads;
  da.nv = c.num_v_heads;
  da.r = ga.r;
  da.Cd = b->cd;
  da.slots = c.num_state_slots;
  da.l2eps = c.l2norm_eps;
  da.geps = c.gated_norm_eps;
  switch (c.head_k_dim) {
    case 32: launch_gdn_d<32>(b, da, rows, st); break;
    case 64: launch_gdn_d<64>(b, da, rows, st); break;
    default: launch_gdn_d<128>(b, da, rows, st); break;
  }
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(b, GDN_E_HIP, std::string("gdn_block_decode: launch failed: ") + hipGetErrorString(e));
  return GDN_OK;
}

extern "C" void gdn_block_destroy(gdn_block_t b) {
  if (!b) return;
  if (b->scratch) (void)hipFree(b->scratch);
  delete b;
}

extern "C" const char* gdn_block_last_error(gdn_block_t b) {
  return b ? b->err.c_str() : g_create_error.c_str();
}
