// Gated DeltaNet decode block for gfx950: one fused decode kernel and the C ABI of
// include/gdn_block.h.
//
// A decode call is ONE launch whose workgroups take one of four roles by block id
// (the front of a GDN layer as one launch, "sgl-amd-mono PR #89", Modifications; the
// "GDN block" of "vLLM PR #60833", Details / Launches):
//
//   [0, R*P)          norm. bf16 and MXFP6 in_proj_qkvz: one workgroup per row (P = 1)
//                     loads the row, forms h = bf16(x + residual) and the row's rstd, and
//                     publishes only the rstd (a word that is never 0, so its own ready
//                     flag); then it rewrites the residual row with h, with a residual
//                     input once every projection workgroup has counted that it loaded its
//                     slice of the row. MXFP4: P = ceil(H / 2048) workgroups per row each
//                     load the whole row (all P sum it in the same order, so with the same
//                     rstd), convert one 2048-wide slice to xn = bf16(h * rstd * (1 + w))
//                     and quantise it to MXFP4 (codes + one e8m0 scale per 32) into a
//                     scratch image, count themselves done and rewrite their residual slice.
//                     No workgroup holds x in LDS ("vLLM PR #60833", Details / x without an
//                     LDS tile). With x already normed there are no norm workgroups, except
//                     MXFP4 past 2 rows: P quantiser workgroups per row make the image.
//   [R*P, R*P+G)      projection: in_proj_qkvz and in_proj_ba as one skinny GEMM on the
//                     matrix cores: bf16 weights on v_mfma_f32_16x16x32_bf16, MXFP4 weights
//                     on v_mfma_scale_f32_16x16x128_f8f6f4 (fp4 x fp4 with per-32 scales),
//                     MXFP6 E2M3 weights converted to bf16 in registers (exactly) and then
//                     on the bf16 instruction with the bf16 activations;
//                     16 weight rows x 16 decode rows per instruction. A workgroup owns one
//                     K range and 4 in_proj_qkvz tiles (one per wave) or one in_proj_ba tile.
//                     It issues its weight loads first (bf16: its last 4 K steps straight
//                     into LDS as well), with bf16 and MXFP6 also the loads of its K range of
//                     x and residual, then waits for the rows' rstd (or the MXFP4 image),
//                     stages the activations of its K range in LDS once, multiplies, and
//                     publishes its f32 partial sums; then it counts itself done for the
//                     tiles' key-head group (or for the b|a tiles).
//   [.., +Rs*nv)      recurrence: one workgroup per (sequence, value head); a decode call
//                     has one token per sequence, a verify call several. It loads its
//                     dk x dv state tile and its conv state and taps first, waits for its
//                     key-head group and the b|a tiles, adds the split partials of its
//                     channels in split order and rounds them to bf16 (the projection
//                     output), runs the causal conv update + SiLU, L2 norms, gates, the gated
//                     delta rule, the state store and the gated RMSNorm into the core output.
//                     A verify step at head dim 128 evaluates its tokens in the chunked form
//                     of the recurrence (rec_verify); below 128 it runs them one after the
//                     other. The q|k conv state of a key head is shared by its r value heads:
//                     the last of them writes it once the others have read the old rows.
//   [.., +H/64)       out_proj (folded in, optional): 4 tiles of 16 hidden columns per
//                     workgroup; the weights stream from launch start, the core rows are
//                     multiplied once every recurrence workgroup has stored its row.
//
// Every wait ends. Projection, recurrence and out_proj workgroups wait only for workgroups
// with lower block ids, which the dispatcher starts first. A norm workgroup's one wait
// (before its residual rewrite) is for workgroups that count themselves before any wait of
// their own and never wait for that rewrite: the projection workgroups, right after loading
// their slice (bf16, MXFP6), or the other norm workgroups (MXFP4). Each wait is also bounded
// and records a sticky error word if it gives up. Data handed from one workgroup to another
// travels as agent-scope stores (coherent across the XCDs' L2s) followed by a wait for the
// stores; readers poll counters with agent-scope atomic loads. No device-wide fence is used:
// on gfx950 one writes back and invalidates a whole L2. Every counter is cleared by the
// last workgroup that reads it, so the next launch starts from zero.
//
// Every reduction runs in a fixed order that does not depend on the row count, so a
// row's results do not change with the other rows (batch invariance, "sgl-amd-mono PR
// #89", Kernel checks).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <mutex>
#include <string>
#include <type_traits>

#include "gdn_block.h"

namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(4))) unsigned u32x4_t;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
typedef __attribute__((ext_vector_type(2))) float f32x2_t;
typedef __attribute__((ext_vector_type(8))) int i32x8_t;
typedef __attribute__((ext_vector_type(2))) unsigned u32x2_t;
typedef __attribute__((ext_vector_type(6))) unsigned u32x6_t;
typedef __attribute__((ext_vector_type(32))) __bf16 bf16x32_t;

// in_proj_qkvz formats (the values of GDN_FMT_*)
constexpr int kFmtBf16 = 0, kFmtMx4 = 1, kFmtMx6 = 2;

constexpr int kConvW = 4;          // conv width; create() refuses any other
constexpr int kThreads = 256;      // every role runs 4 waves of 64
constexpr int kLine = 32;          // uint32 words per 128-byte line: one hot counter per line
// Weight loads each wave keeps in flight (1 KiB each). The window is refilled as it is
// consumed: enough bytes in flight to keep HBM busy, few enough that the hand-offs between
// workgroups are not queued behind the whole weight matrix. Measured at the TP8-rank shape:
// 8 beats 2, 4 and 6, and also 12, 16 and 24 (deeper windows slow the stream itself).
#ifndef GDN_WINDOW
#define GDN_WINDOW 8
#endif
constexpr int kWin = GDN_WINDOW;
constexpr int kSpinLimit = 1 << 20;  // default poll limit of a bounded wait (Args::spin)
constexpr int kNormCopies = 8;     // the norm-done counter is kept on 8 lines, polled spread out
constexpr int kGroupCopies = 8;    // a key-head group's tiles-done counter is spread over 8 lines
constexpr int kCoreCopies = 16;    // so is the core-done counter of the out_proj fold, on 16

// ---------------------------------------------------------------------------------------
// scalar helpers

__device__ __forceinline__ float bf2f(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// f32 -> bf16, round to nearest even: gfx950 converts in hardware (v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint16_t f2bf(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }
// two values at once: lo in the low half, hi in the high half
__device__ __forceinline__ uint32_t f2bf2(float lo, float hi) {
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

__device__ __forceinline__ float rbf(float f) { return bf2f(f2bf(f)); }  // the bf16 value of f

__device__ __forceinline__ float silu(float x) { return x * __builtin_amdgcn_rcpf(1.0f + __expf(-x)); }

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

// Cross-lane exchanges on the VALU instead of the LDS crossbar. dpp<CTRL>(v): v from the
// lane that the DPP control picks (row_ror:8 = 0x128, a rotation by 8 within each row of 16
// lanes, is the xor-8 partner; quad_perm [1,0,3,2] = 0xB1 and [2,3,0,1] = 0x4E the xor-1
// and xor-2 partners; row_half_mirror = 0x141 pairs lane i with 7 - i within 8 lanes).
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
// v[e] += (v[e] in lane ^ M) for e < 4, M = 16 or 32, with gfx950's v_permlane16_swap /
// v_permlane32_swap: swapping a copy of v with another copy leaves each lane's xor
// partner in one of the two (rows 2j+1 with rows 2j of the other, or the upper half with
// the lower half). Inline asm, padded with s_nop on both sides: a swap that reads a VGPR
// the previous VALU instruction wrote reads its old value (measured on MI355X), and the
// compiler does not insert wait states for inline asm.
template <int M>
__device__ __forceinline__ void xor_add4(float& v0, float& v1, float& v2, float& v3) {
  float a0 = v0, b0 = v0, a1 = v1, b1 = v1, a2 = v2, b2 = v2, a3 = v3, b3 = v3;
  if constexpr (M == 16)
    asm volatile(
        "s_nop 4\n\tv_permlane16_swap_b32 %0, %1\n\tv_permlane16_swap_b32 %2, %3\n\t"
        "v_permlane16_swap_b32 %4, %5\n\tv_permlane16_swap_b32 %6, %7\n\ts_nop 4"
        : "+v"(a0), "+v"(b0), "+v"(a1), "+v"(b1), "+v"(a2), "+v"(b2), "+v"(a3), "+v"(b3));
  else
    asm volatile(
        "s_nop 4\n\tv_permlane32_swap_b32 %0, %1\n\tv_permlane32_swap_b32 %2, %3\n\t"
        "v_permlane32_swap_b32 %4, %5\n\tv_permlane32_swap_b32 %6, %7\n\ts_nop 4"
        : "+v"(a0), "+v"(b0), "+v"(a1), "+v"(b1), "+v"(a2), "+v"(b2), "+v"(a3), "+v"(b3));
  // the partner is in a for the odd row (M = 16) or upper half (M = 32), else in b
  const bool hi = (threadIdx.x & M) != 0;
  v0 += hi ? a0 : b0;
  v1 += hi ? a1 : b1;
  v2 += hi ? a2 : b2;
  v3 += hi ? a3 : b3;
}
// v[e] += (v[e] in lane ^ M) for every e, M a power of two below 64; each pair adds the
// same two values (in either order), so both lanes hold the same sum
template <int M, int N>
__device__ __forceinline__ void xor_add(float (&v)[N]) {
  if constexpr (M == 16 || M == 32) {
#pragma unroll
    for (int e = 0; e < N; e += 4) {
      float d0 = 0.0f, d1 = 0.0f, d2 = 0.0f;
      xor_add4<M>(v[e], e + 1 < N ? v[e + 1] : d0, e + 2 < N ? v[e + 2] : d1, e + 3 < N ? v[e + 3] : d2);
    }
  } else {
#pragma unroll
    for (int e = 0; e < N; ++e) v[e] += M == 8 ? dpp<0x128>(v[e]) : __shfl_xor(v[e], M, 64);
  }
}
// the xor butterfly over lane bits M, 2M, ... 32: every lane ends with the sum over its
// 64 / M lanes that agree with it on the bits below M
template <int M, int N>
__device__ __forceinline__ void xor_butterfly(float (&v)[N]) {
  if constexpr (M < 64) {
    xor_add<M>(v);
    xor_butterfly<2 * M>(v);
  }
}

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t v) { return __builtin_bit_cast(bf16x8_t, v); }

__device__ __forceinline__ uint32_t pack2(uint16_t lo, uint16_t hi) { return (uint32_t)lo | ((uint32_t)hi << 16); }

// cross-workgroup hand-off: single accesses coherent at agent scope
__device__ __forceinline__ void st_agent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_agent(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_agent(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t ld_agent(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t add_agent(uint32_t* p, uint32_t v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// this wave's loads have returned and its stores have completed (so a counter bumped
// after them is seen after them)
__device__ __forceinline__ void wait_stores() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
// s_waitcnt immediate for vmcnt(0) alone (gfx9 encoding: vmcnt 0, expcnt 7, lgkmcnt 15). As
// a builtin (not asm) the compiler's own wait placement sees it: registers loaded before it
// are then known ready, where it would otherwise wait for every memory operation in flight
// at their first use, stores included.
constexpr int kWaitVm0 = 0x0F70;
// 16-byte store coherent at agent scope (the vector form of st_agent)
__device__ __forceinline__ void st_agent16(uint32_t* p, u32x4_t v) {
  asm volatile("global_store_dwordx4 %0, %1, off sc1" ::"v"(p), "v"(v) : "memory");
}

// The whole workgroup waits until a counter reaches `target`. Wave 0 polls, backing off
// between polls so that waiting workgroups do not crowd the counter's memory channel;
// it gives up after `limit` polls, recording `code`. No memory access after the call
// is moved above it.
__device__ __forceinline__ void wait_count(uint32_t* ctr, uint32_t target, uint32_t* err, uint32_t code, int limit) {
  if (threadIdx.x < 64) {
    int it = 0;
    while (ld_agent(ctr) < target) {
      __builtin_amdgcn_s_sleep(4);
      if (++it > limit) {
        __hip_atomic_fetch_or(err, code, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
    }
  }
  __syncthreads();
  asm volatile("" ::: "memory");
}

// In-kernel timeline for profiling builds (-DGDN_TRACE): thread 0 of each workgroup stamps
// the 100 MHz wall clock at up to kTraceSlots points of its role. Compiled out otherwise.
#ifdef GDN_TRACE
constexpr int kTraceSlots = 16;
constexpr int kTraceBlocks = 8192;
__device__ unsigned long long g_trace[kTraceBlocks * kTraceSlots];
#define TRACE_POINT(k)                                                                          \
  do {                                                                                          \
    if (threadIdx.x == 0 && blockIdx.x < kTraceBlocks) g_trace[blockIdx.x * kTraceSlots + (k)] = wall_clock64(); \
  } while (0)
// slot k <- (XCC id << 32) | hardware id word (CU, SE, ...) of the wave
#define TRACE_HWID(k)                                                                           \
  do {                                                                                          \
    if (threadIdx.x == 0 && blockIdx.x < kTraceBlocks)                                          \
      g_trace[blockIdx.x * kTraceSlots + (k)] =                                                 \
          ((unsigned long long)__builtin_amdgcn_s_getreg((3 << 11) | 20) << 32) |              \
          (unsigned long long)__builtin_amdgcn_s_getreg((31 << 11) | 4);                        \
  } while (0)
#else
#define TRACE_POINT(k) \
  do {                 \
  } while (0)
#define TRACE_HWID(k) \
  do {                \
  } while (0)
#endif

// sync word lines (one 128-byte line each): norm workgroups done (kNormCopies copies,
// polled spread out; the MXFP4 path); b|a tile splits done; recurrence workgroups
// finished; the sticky error word; norm workgroups finished; out_proj workgroups past
// their wait and (on kCoreCopies lines) recurrence workgroups whose core rows are stored
// (out_proj fold); each row's rstd, on kNormCopies lines (word r of a line is row r's
// rstd, 0 until published); projection workgroups holding their residual slice, on
// kNormCopies lines; then per key-head group, on kGroupCopies lines: tile splits done;
// then per (sequence, key-head group): value heads that have read the old q|k conv rows.
enum {
  kSyNorm = 0,
  kSyBa = kNormCopies,
  kSyExit,
  kSyError,
  kSyNormExit,
  kSyOutExit,  // top line of the out_proj workgroups' two-level exit count
  kSyCoreDone,
  kSyOutExit1 = kSyCoreDone + kCoreCopies,  // its first level, kCoreCopies lines
  kSyRstd = kSyOutExit1 + kCoreCopies,
  kSyLoaded = kSyRstd + kNormCopies,
  kSyGroup0 = kSyLoaded + kNormCopies
};
enum : uint32_t { kErrNormWait = 1u, kErrGroupWait = 2u, kErrConvWait = 4u };

// ---------------------------------------------------------------------------------------

struct Args {
  // caller tensors
  const uint16_t* x;         // [R, H]
  uint16_t* residual;        // [R, H] in/out
  const uint16_t* norm_w;    // [H]
  const uint16_t* wq;        // in_proj_qkvz [Nq, H] (row-major path)
  const uint16_t* wb;        // in_proj_ba [Nb, H] (row-major path)
  const uint16_t* wpk;       // tiled copy: in_proj_qkvz tiles (bf16, or MXFP4 codes)
  const uint16_t* wpk_ba;    // tiled copy: in_proj_ba tiles (bf16)
  const uint8_t* wqc;        // MXFP4 in_proj_qkvz codes [Nq, H/2] (row-major path)
  const uint8_t* wqs;        // MXFP4 in_proj_qkvz scales [Nq, H/32] (row-major path)
  const uint32_t* wpk_sc;    // tiled copy: MXFP4 scales, one dword per lane per 4 K steps
  const uint16_t* conv_w;    // [Cd, 4]
  uint16_t* conv_state;      // [slots, 3, Cd]
  void* ssm;                 // [slots, nv, dk, dv] f32 or bf16
  const int32_t* idx;        // [Rs] each sequence's state slot (decode: one token per sequence)
  const int32_t* dst;        // [Rs, Tk] slots that receive the state after each token (verify), or null
  const float* A_log;        // [nv]
  const uint16_t* dt_bias;   // [nv]
  const uint16_t* gnw;       // [dv]
  uint16_t* core;            // [R, nv*dv]
  const uint16_t* wo;        // out_proj [H, nv*dv] (row-major path, fold only)
  const uint16_t* wo_pk;     // out_proj tiles (packed path, fold only)
  uint16_t* out;             // [R, H] the out_proj partial (fold only)
  // scratch
  uint16_t* xn;              // [R, H]
  uint32_t* xq;              // MXFP4 image of xn: codes [R, H/2] bytes
  uint32_t* xqs;             // MXFP4 image of xn: scales [R, H/32] bytes, grouped per 4 K steps
  float* part;               // [S, R, Nq + Nb] split partials of the projections
  uint32_t* sync;            // sync word lines
  // sizes
  int H, R, has_res, P;  // R: token rows (Rs sequences x Tk tokens); P: norm workgroups per row
  int Rs, Tk;            // sequences and tokens per sequence (decode: Tk = 1)
  int normed;            // x is already the norm's output xn
  int fold, O, Ko;       // out_proj folded in; its workgroups (4 16-column tiles of H each); K = nv*dv
  int T, Tq, Tb, Nq, Nb, steps;  // tiles (all, in_proj_qkvz, in_proj_ba), channels, 32-wide K steps of H
  int S, Kr, G, Gq;              // K ranges (splits) of Kr each, projection workgroups, of which
                                 // in_proj_qkvz ones
  int nk, dk, nv, dv, r, GW, Cd, slots;
  int PW;      // floats per row of the split partials: Nq + Nb rounded up to whole 128-byte lines
  int spin;    // poll limit of every bounded wait
  int mx_ceil; // MXFP4 activation scale rule: 0 rounded maximum, 1 ceiling
  int wlds;    // bf16 projections fetch their last weight steps into LDS at launch (1) or not
  float eps, l2eps, geps;
};

__device__ __forceinline__ uint32_t* sy(const Args& a, int line) { return a.sync + (size_t)line * kLine; }
__device__ __forceinline__ int sy_group(int g, int c) { return kSyGroup0 + g * kGroupCopies + c; }
__device__ __forceinline__ int sy_conv(const Args& a, int n, int g) {
  return kSyGroup0 + a.nk * kGroupCopies + n * a.nk + g;
}

// ---------------------------------------------------------------------------------------
// role 1: residual add + Gemma RMSNorm of one row

constexpr int kNormMaxChunks = 8;  // 16-byte chunks per thread: H <= 8 * 8 * 256

// MXFP4 quantisation of one 32-element block held by 4 consecutive lanes, 8 bf16 each
// (dwords in element order, the even element in the low half) ("vLLM PR #60833", Details
// / MoE: dynamic MXFP4 in 1x32 blocks; Details / MXFP4 layouts: two roundings of the
// scale). With max|x| = M * 2^E (1 <= M < 2, read off the bf16 bits of the maximum) the
// block exponent e is E - 2 plus a carry, clamped below at -126 (a zero or subnormal
// maximum gives -126):
//   ceil == 0, the rounded maximum (the same page's account of dynamic_mxfp4_quant, in the
//     reviewer's comment proposing MXFP6): M rounded half up at e2m1's one mantissa bit
//     carries when M >= 1.75, i.e. when the top two of the 7 mantissa bits are set;
//   ceil == 1, the smallest e with max|x| <= 6 * 2^e: a carry when M > 1.5.
// Each x / 2^e (exact: a power-of-two scaling) is rounded to the nearest e2m1 value, ties
// to the even code: the code counts the rounding boundaries 0.25, 0.75, 1.25, 1.75, 2.5,
// 3.5, 5 that |x| / 2^e passes (a boundary that is a tie belongs to the even side); a value
// past 6 (up to 7 with the rounded maximum) takes the top code. A zero code carries no
// sign. All 4 lanes of the block must be active. Returns the 8 codes (element 8 j + q in
// nibble q); the scale byte e + 127 goes to `ebyte`.
__device__ __forceinline__ uint32_t mx_quant8(const uint32_t* v, uint32_t& ebyte, int ceil) {
  uint32_t m = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) m = max(m, max(v[q] & 0x7fffu, (v[q] >> 16) & 0x7fffu));
  m = max(m, (uint32_t)__shfl_xor((int)m, 1, 64));
  m = max(m, (uint32_t)__shfl_xor((int)m, 2, 64));
  const int ef = (int)(m >> 7);
  const uint32_t mant = m & 0x7fu;
  const int carry = ceil ? (mant > 0x40u ? 1 : 0) : (mant >= 0x60u ? 1 : 0);
  const int e = ef == 0 ? -126 : max(-126, ef - 129 + carry);
  const float inv = __uint_as_float((uint32_t)(127 - e) << 23);  // 2^-e
  uint32_t codes = 0;
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const uint32_t b = (q & 1) ? (v[q >> 1] >> 16) : (v[q >> 1] & 0xffffu);
    const float x = bf2f((uint16_t)(b & 0x7fffu)) * inv;
    uint32_t c = (uint32_t)(x > 0.25f) + (uint32_t)(x >= 0.75f) + (uint32_t)(x > 1.25f) + (uint32_t)(x >= 1.75f) +
                 (uint32_t)(x > 2.5f) + (uint32_t)(x >= 3.5f) + (uint32_t)(x > 5.0f);
    if ((b & 0x8000u) && c) c |= 8u;
    codes |= c << (4 * q);
  }
  ebyte = (uint32_t)(e + 127);
  return codes;
}

// Without MXFP4 (bf16 or MXFP6 in_proj_qkvz): one workgroup per row loads the whole row,
// forms h = bf16(x + residual) and the row's rstd, and publishes only rstd, as the data
// itself: word `row` of kNormCopies lines, 0 until written (rstd is never 0). Projection
// workgroups load the x (and residual) slice of their own K range at launch and form xn
// from it with the same arithmetic once rstd is there, so no xn row makes a round trip
// through memory ("vLLM PR #60833", Details: x is not held in LDS; rstd is handed off).
// The residual row is then rewritten with h: with a residual input, only once every
// projection workgroup holds its residual slice.
__device__ void norm_rstd_role(const Args& a, int row, float* red) {
  const int H = a.H, nchunk = H >> 3, tid = threadIdx.x;
  const uint4* xp = reinterpret_cast<const uint4*>(a.x + (size_t)row * H);
  uint4* rp = reinterpret_cast<uint4*>(a.residual + (size_t)row * H);
  uint4 hv[kNormMaxChunks], rv[kNormMaxChunks];
#pragma unroll
  for (int c = 0; c < kNormMaxChunks; ++c) {  // every load of the row is issued up front
    const int i = tid + c * kThreads;
    if (i < nchunk) hv[c] = xp[i];
  }
  if (a.has_res) {
#pragma unroll
    for (int c = 0; c < kNormMaxChunks; ++c) {
      const int i = tid + c * kThreads;
      if (i < nchunk) rv[c] = rp[i];
    }
  }
  float ss = 0.0f;
#pragma unroll
  for (int c = 0; c < kNormMaxChunks; ++c) {
    const int i = tid + c * kThreads;
    if (i < nchunk) {
      if (a.has_res) {
        uint32_t* pv = reinterpret_cast<uint32_t*>(&hv[c]);
        const uint32_t* pb = reinterpret_cast<const uint32_t*>(&rv[c]);
#pragma unroll
        for (int k = 0; k < 4; ++k)
          pv[k] = f2bf2(bf2f((uint16_t)pv[k]) + bf2f((uint16_t)pb[k]),
                        bf2f((uint16_t)(pv[k] >> 16)) + bf2f((uint16_t)(pb[k] >> 16)));
      }
      const uint32_t* ph = reinterpret_cast<const uint32_t*>(&hv[c]);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float l = bf2f((uint16_t)ph[k]), h = bf2f((uint16_t)(ph[k] >> 16));
        ss = fmaf(l, l, ss);
        ss = fmaf(h, h, ss);
      }
    }
  }
  ss = block_sum(ss, red);
  TRACE_POINT(1);
  const float rstd = 1.0f / sqrtf(ss / (float)H + a.eps);
  if (tid < kNormCopies) st_agent(reinterpret_cast<float*>(sy(a, kSyRstd + tid)) + row, rstd);
  TRACE_POINT(2);
  if (a.has_res) {
    // every projection workgroup has counted itself on line gb % kNormCopies once it holds
    // its residual slice: lane c of the first wave waits for line c's share
    if (threadIdx.x < 64) {
      const int c = threadIdx.x;
      const int share = c < kNormCopies ? max(0, (a.G - c + kNormCopies - 1) / kNormCopies) : 0;
      uint32_t* ctr = sy(a, kSyLoaded + (c < kNormCopies ? c : 0));
      int it = 0;
      while (!__all(share == 0 || ld_agent(ctr) >= (uint32_t)share)) {
        __builtin_amdgcn_s_sleep(8);
        if (++it > a.spin) {
          if (c == 0) __hip_atomic_fetch_or(sy(a, kSyError), kErrNormWait, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          break;
        }
      }
    }
    __syncthreads();
    asm volatile("" ::: "memory");
  }
#pragma unroll
  for (int c = 0; c < kNormMaxChunks; ++c) {
    const int i = tid + c * kThreads;
    if (i < nchunk) rp[i] = hv[c];
  }
  wait_stores();
  __syncthreads();
  if (tid == 0) add_agent(sy(a, kSyNormExit), 1u);
  TRACE_POINT(3);
}

// MXFP4 image of one 2048-wide slice of a row (8 bf16 per thread): codes and the grouped
// scale dwords, stored coherently for the projection workgroups
__device__ __forceinline__ void store_image(const Args& a, int row, int mi, const u32x4_t& o4) {
  const int H = a.H, tid = threadIdx.x;
  // H is a multiple of 512, so a wave's 64 chunks are all in range together
  uint32_t v[4] = {o4[0], o4[1], o4[2], o4[3]}, eb;
  st_agent(a.xq + (size_t)row * (H >> 3) + mi, mx_quant8(v, eb, a.mx_ceil));
  // The wave's 64 chunks are the 16 blocks of 4 K steps of 128: block 4 s + kb holds
  // K quarter kb of step s. Scales are stored per (4 steps, quarter kb) as one dword,
  // byte s, the operand a projection lane of quarter kb reads for 4 steps at once.
  const int lane = tid & 63, kb = (lane >> 2) & 3;
  uint32_t d = 0;
#pragma unroll
  for (int st = 0; st < 4; ++st) d |= (uint32_t)__shfl((int)eb, 16 * st + 4 * kb, 64) << (8 * st);
  if (lane < 16 && (lane & 3) == 0) st_agent(a.xqs + (size_t)row * (H >> 7) + 4 * (mi >> 6) + kb, d);
}

// With a normed input and MXFP4 at more than 2 rows: P workgroups per row quantise x (which
// is xn) once, 2048 columns each, into the shared image, instead of every projection
// workgroup quantising its K range of every row (measured faster from 3 rows on).
__device__ void quant_role(const Args& a, int b) {
  const int row = b / a.P, part = b - row * a.P, mi = part * kThreads + threadIdx.x;
  if (mi < (a.H >> 3)) {
    const uint4 q = reinterpret_cast<const uint4*>(a.x + (size_t)row * a.H)[mi];
    store_image(a, row, mi, u32x4_t{q.x, q.y, q.z, q.w});
  }
  wait_stores();
  __syncthreads();
  if (threadIdx.x < kNormCopies) add_agent(sy(a, kSyNorm + threadIdx.x), 1u);
  if (threadIdx.x == 0) add_agent(sy(a, kSyNormExit), 1u);
}

template <bool MX>
__device__ void norm_role(const Args& a, int b, float* red) {
  // P workgroups per row: each loads and sums the whole row (the same sum in the same
  // order, so the same rstd in all of them) and produces xn for one slice of 256 chunks
  // of 8 elements, so no thread converts more than one chunk
  const int row = b / a.P, part = b - row * a.P;
  const int H = a.H, nchunk = H >> 3, tid = threadIdx.x;
  const uint4* xp = reinterpret_cast<const uint4*>(a.x + (size_t)row * H);
  uint4* rp = reinterpret_cast<uint4*>(a.residual + (size_t)row * H);
  const int mi = part * kThreads + tid;  // this thread's chunk of the slice
  uint4 hv[kNormMaxChunks], rv[kNormMaxChunks], wv = make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
  for (int c = 0; c < kNormMaxChunks; ++c) {  // every load of the row is issued up front
    const int i = tid + c * kThreads;
    if (i < nchunk) hv[c] = xp[i];
  }
  if (a.has_res) {
#pragma unroll
    for (int c = 0; c < kNormMaxChunks; ++c) {
      const int i = tid + c * kThreads;
      if (i < nchunk) rv[c] = rp[i];
    }
  }
  if (mi < nchunk) wv = reinterpret_cast<const uint4*>(a.norm_w)[mi];
  float ss = 0.0f;
  uint4 mine = make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
  for (int c = 0; c < kNormMaxChunks; ++c) {
    const int i = tid + c * kThreads;
    if (i < nchunk) {
      uint4 v = hv[c];
      if (a.has_res) {
        const uint4 q = rv[c];
        uint32_t* pv = reinterpret_cast<uint32_t*>(&v);
        const uint32_t* pb = reinterpret_cast<const uint32_t*>(&q);
#pragma unroll
        for (int k = 0; k < 4; ++k)
          pv[k] = f2bf2(bf2f((uint16_t)pv[k]) + bf2f((uint16_t)pb[k]),
                        bf2f((uint16_t)(pv[k] >> 16)) + bf2f((uint16_t)(pb[k] >> 16)));
      }
      if (c == part) mine = v;
      const uint32_t* ph = reinterpret_cast<const uint32_t*>(&v);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float l = bf2f((uint16_t)ph[k]), h = bf2f((uint16_t)(ph[k] >> 16));
        ss = fmaf(l, l, ss);
        ss = fmaf(h, h, ss);
      }
    }
  }
  ss = block_sum(ss, red);
  TRACE_POINT(1);
  const float rstd = 1.0f / sqrtf(ss / (float)H + a.eps);
  if (mi < nchunk) {
    const uint32_t* ph = reinterpret_cast<const uint32_t*>(&mine);
    const uint32_t* pw = reinterpret_cast<const uint32_t*>(&wv);
    u32x4_t o4;
#pragma unroll
    for (int k = 0; k < 4; ++k)
      o4[k] = f2bf2(bf2f((uint16_t)ph[k]) * rstd * (1.0f + bf2f((uint16_t)pw[k])),
                    bf2f((uint16_t)(ph[k] >> 16)) * rstd * (1.0f + bf2f((uint16_t)(pw[k] >> 16))));
    st_agent16(reinterpret_cast<uint32_t*>(a.xn + (size_t)row * H) + 4 * mi, o4);
    if (MX) store_image(a, row, mi, o4);
  }
  TRACE_POINT(2);
  wait_stores();
  __syncthreads();
  if (tid < kNormCopies) add_agent(sy(a, kSyNorm + tid), 1u);
  // The residual row is rewritten with h, each workgroup its own slice. With a residual
  // input every workgroup of the row reads the whole row first: the rewrite waits until
  // every norm workgroup has counted itself (so has finished loading).
  if (a.has_res) wait_count(sy(a, kSyNorm + b % kNormCopies), (uint32_t)(a.R * a.P), sy(a, kSyError), kErrNormWait, a.spin);
  if (mi < nchunk) rp[mi] = mine;
  wait_stores();
  __syncthreads();
  if (tid == 0) add_agent(sy(a, kSyNormExit), 1u);
  TRACE_POINT(3);
}

// ---------------------------------------------------------------------------------------
// role 2: one split of one 16-channel projection tile

// A projection workgroup owns one K range of Kr (<= kKr) and either 4 in_proj_qkvz tiles
// (one per wave, each over the whole range) or one in_proj_ba tile (its 4 waves taking a
// quarter of the range each). It stages the activations of its K range (the xn slice, or
// the MXFP4 image of it) in LDS once, so they cross the load path once per workgroup
// instead of once per tile, and every wave reads its operand from LDS.
constexpr int kKr = 1024;   // largest K range of a projection workgroup
constexpr int kXPad = 8;    // bf16 of padding per LDS row, so that the 16 rows start on different banks
constexpr int kMxRow = kKr / 2 + 16;         // LDS bytes per row of MXFP4 codes (padded)
constexpr int kMxScBase = GDN_MAX_ROWS * kMxRow;  // LDS byte offset of the MXFP4 scale rows

constexpr int kLdsSteps = 4;  // bf16 weight steps per wave fetched straight into LDS at launch
struct ProjShared {
  uint16_t xs[GDN_MAX_ROWS][kKr + kXPad];  // the activation slice [decode row][k], or MXFP4 image bytes
  float red[4][256];
  u32x4_t wl[4][kLdsSteps][64];  // per wave: the last kLdsSteps weight steps of its range
};

// the 4 waves' accumulators of one tile -> the tile's split partials (fixed-order sum over
// the waves), then the tile counts itself done. D layout of the 16x16 MFMAs: lane l holds
// channels 4 (l / 16) + i (i = 0..3) of decode row l % 16.
__device__ __forceinline__ void publish_reduced(const Args& a, int t, int s, f32x4_t acc, float (*red)[256]) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, tid = threadIdx.x;
  const bool isq = t < a.Tq;
#pragma unroll
  for (int i = 0; i < 4; ++i) red[wave][i * 64 + lane] = acc[i];
  __syncthreads();
  const int en = tid >> 4, em = tid & 15;  // this thread's (decode row, channel) of the tile
  const int src = (em & 3) * 64 + (em >> 2) * 16 + en;
  const float v = ((red[0][src] + red[1][src]) + red[2][src]) + red[3][src];
  const int ch = (isq ? t * 16 : a.Nq + (t - a.Tq) * 16) + em;  // channel in [qkvz | ba] order
  if (en < a.R && (isq || ch < a.Nq + a.Nb)) st_agent(&a.part[((size_t)s * a.R + en) * a.PW + ch], v);
  wait_stores();
  __syncthreads();
  if (tid == 0) add_agent(sy(a, kSyBa), 1u);  // only b|a tiles are published this way
}

// each wave's own in_proj_qkvz tile -> its split partials; then the 4 tiles (one key-head
// group never straddles a workgroup's tiles) count as one
__device__ __forceinline__ void publish_tiles(const Args& a, int t0, int s, f32x4_t acc) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int en = lane & 15;
  if (en < a.R) {  // the lane's 4 channels are adjacent: one 16-byte store
    const int ch = (t0 + wave) * 16 + 4 * (lane >> 4);
    const u32x4_t v = {__float_as_uint(acc[0]), __float_as_uint(acc[1]), __float_as_uint(acc[2]), __float_as_uint(acc[3])};
    st_agent16(reinterpret_cast<uint32_t*>(&a.part[((size_t)s * a.R + en) * a.PW + ch]), v);
  }
  wait_stores();
  __syncthreads();
  // The group's tile workgroups count themselves on kGroupCopies lines (one line takes the
  // atomics one at a time: ~96 arriving together would queue for about a microsecond).
  // Workgroup li of the group (tile group, then split) counts on line li % kGroupCopies.
  if (threadIdx.x == 0) {
    const int g = t0 * 16 / a.GW, li = (t0 / 4 - g * (a.GW / 64)) * a.S + s;
    add_agent(sy(a, sy_group(g, li % kGroupCopies)), 1u);
  }
}

// waits until every tile workgroup of key-head group g has counted itself: lane c of the
// first wave polls line c for its share, (n - c + C - 1) / C of the group's n workgroups
__device__ __forceinline__ void wait_group(const Args& a, int g) {
  if (threadIdx.x < 64) {
    const int c = threadIdx.x, n = a.GW / 64 * a.S;
    const int share = c < kGroupCopies ? max(0, (n - c + kGroupCopies - 1) / kGroupCopies) : 0;
    uint32_t* ctr = sy(a, sy_group(g, c < kGroupCopies ? c : 0));
    int it = 0;
    while (!__all(share == 0 || ld_agent(ctr) >= (uint32_t)share)) {
      __builtin_amdgcn_s_sleep(4);
      if (++it > a.spin) {
        if (c == 0) __hip_atomic_fetch_or(sy(a, kSyError), kErrGroupWait, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
    }
  }
  __syncthreads();
  asm volatile("" ::: "memory");
}

// bf16 weight operand of local K step l (32 wide) of K range s for this lane: 8 bf16 of row
// (lane % 16) at k = s Kr + 32 l + 8 (lane / 16). In the tiled copy a step of a tile is one
// 1 KiB block in lane order; in_proj_qkvz blocks are grouped as [K range][group of 4 tiles]
// [step][tile of the group], so the 4 waves of a projection workgroup read 4 adjacent
// blocks at each step and the workgroup's whole share is one contiguous run (measured 4 %
// faster to stream than one run per tile); in_proj_ba tiles keep one run per tile.
template <bool PACKED>
__device__ __forceinline__ const u32x4_t* wptr(const Args& a, int t, int s, int l, int lane) {
  const bool isq = t < a.Tq;
  const int ns = a.Kr >> 5;  // steps per K range
  if (PACKED) {
    if (isq)
      return reinterpret_cast<const u32x4_t*>(
          a.wpk + ((((size_t)s * (a.Tq >> 2) + (t >> 2)) * ns + l) * 4 + (t & 3)) * 512 + (size_t)lane * 8);
    return reinterpret_cast<const u32x4_t*>(a.wpk_ba + ((size_t)(t - a.Tq) * a.steps + s * ns + l) * 512 +
                                            (size_t)lane * 8);
  }
  const int N = isq ? a.Nq : a.Nb;
  // rows past the end are clamped to valid memory; their outputs are never stored
  const int row = min((isq ? t : t - a.Tq) * 16 + (lane & 15), N - 1);
  return reinterpret_cast<const u32x4_t*>((isq ? a.wq : a.wb) + (size_t)row * a.H + 32 * (s * ns + l) +
                                          8 * (lane >> 4));
}

// waits for the norm rows, then copies xn[0..R)[k0, k0 + Kr) into LDS
__device__ __forceinline__ void stage_xn(const Args& a, int gb, int k0, ProjShared& sh) {
  wait_count(sy(a, kSyNorm + gb % kNormCopies), (uint32_t)(a.R * a.P), sy(a, kSyError), kErrNormWait, a.spin);
  TRACE_POINT(1);
  // 16-byte chunks: cpr per row (<= 128), so each pass of the workgroup covers rpp >= 2 rows
  const int cpr = a.Kr >> 3, rpp = kThreads / cpr, r0 = threadIdx.x / cpr, q = threadIdx.x - r0 * cpr;
  const bool on = r0 < rpp;
  constexpr int kPass = GDN_MAX_ROWS / 2;
  // two rounds of up to 4 loads in flight per thread, so the copy keeps few registers
#pragma unroll 1
  for (int u0 = 0; u0 < kPass; u0 += 4) {
    u32x4_t v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int row = r0 + (u0 + u) * rpp;
      if (on && row < a.R) v[u] = *reinterpret_cast<const u32x4_t*>(a.xn + (size_t)row * a.H + k0 + 8 * q);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int row = r0 + (u0 + u) * rpp;
      if (on && row < a.R) *reinterpret_cast<u32x4_t*>(&sh.xs[row][8 * q]) = v[u];
    }
  }
  __syncthreads();
}

// A normed input (x is xn): no workgroup waits for another before its first multiply. The
// projection workgroup issues the loads of its K range of x before its weight loads, so
// they return first, and stores them to LDS (bf16), or quantises them into the MXFP4 image
// there ("SGLang PR #43558", Modifications: the normed build, every CTA quantising the
// rows itself). MXFP4 past 2 rows instead reads the image the quantiser workgroups make
// once per row: quantising every row in every workgroup costs more there than the wait.
constexpr int kXnChunks = GDN_MAX_ROWS * kKr / 8 / kThreads;  // 16-byte chunks per thread at most
struct XnIn {
  u32x4_t v[kXnChunks];
};
// bf16: chunk (row r0 + u rpp, column chunk q) per thread, as stage_xn maps them
__device__ __forceinline__ void xin_issue(const Args& a, int k0, XnIn& in) {
  const int cpr = a.Kr >> 3, rpp = kThreads / cpr, r0 = threadIdx.x / cpr, q = threadIdx.x - r0 * cpr;
#pragma unroll
  for (int u = 0; u < kXnChunks; ++u) {
    const int row = r0 + u * rpp;
    if (r0 < rpp && row < a.R) in.v[u] = *reinterpret_cast<const u32x4_t*>(a.x + (size_t)row * a.H + k0 + 8 * q);
  }
}
__device__ __forceinline__ void xin_store(const Args& a, const XnIn& in, ProjShared& sh) {
  const int cpr = a.Kr >> 3, rpp = kThreads / cpr, r0 = threadIdx.x / cpr, q = threadIdx.x - r0 * cpr;
#pragma unroll
  for (int u = 0; u < kXnChunks; ++u) {
    const int row = r0 + u * rpp;
    if (r0 < rpp && row < a.R) *reinterpret_cast<u32x4_t*>(&sh.xs[row][8 * q]) = in.v[u];
  }
  __syncthreads();
  TRACE_POINT(1);
}
// Without MXFP4 the norm hands off only each row's rstd (norm_rstd_role). A projection
// workgroup loads the x slice [0, R) x [k0, k0 + Kr) (and the residual slice) and its slice
// of the norm weight at launch, before its weight loads, in the chunk mapping of
// xin_issue; stage_h turns them into the xn slice in LDS.
struct HIn {
  XnIn x, r;
  u32x4_t w;  // norm weight of this thread's 8 columns
};
__device__ __forceinline__ void hin_issue(const Args& a, int k0, HIn& in) {
  const int cpr = a.Kr >> 3, rpp = kThreads / cpr, r0 = threadIdx.x / cpr, q = threadIdx.x - r0 * cpr;
  if (r0 >= rpp) return;
#pragma unroll
  for (int u = 0; u < kXnChunks; ++u) {
    const int row = r0 + u * rpp;
    if (row < a.R) in.x.v[u] = *reinterpret_cast<const u32x4_t*>(a.x + (size_t)row * a.H + k0 + 8 * q);
  }
  if (a.has_res) {
#pragma unroll
    for (int u = 0; u < kXnChunks; ++u) {
      const int row = r0 + u * rpp;
      if (row < a.R) in.r.v[u] = *reinterpret_cast<const u32x4_t*>(a.residual + (size_t)row * a.H + k0 + 8 * q);
    }
  }
  in.w = *reinterpret_cast<const u32x4_t*>(a.norm_w + k0 + 8 * q);
}
// h = bf16(x + residual) (or x) into LDS; with a residual input the workgroup then counts
// itself as holding its residual slice (the LDS writes need the loaded data, so after the
// barrier every load of the slice has returned); waits for the rows' rstd; and converts
// its chunks to xn = bf16(h * rstd * (1 + w)) in place, the norm's own arithmetic.
__device__ __forceinline__ void stage_h(const Args& a, int gb, const HIn& in, ProjShared& sh) {
  const int cpr = a.Kr >> 3, rpp = kThreads / cpr, r0 = threadIdx.x / cpr, q = threadIdx.x - r0 * cpr;
  const bool on = r0 < rpp;
#pragma unroll
  for (int u = 0; u < kXnChunks; ++u) {
    const int row = r0 + u * rpp;
    if (on && row < a.R) {
      u32x4_t h = in.x.v[u];
      if (a.has_res) {
#pragma unroll
        for (int k = 0; k < 4; ++k)
          h[k] = f2bf2(bf2f((uint16_t)h[k]) + bf2f((uint16_t)in.r.v[u][k]),
                       bf2f((uint16_t)(h[k] >> 16)) + bf2f((uint16_t)(in.r.v[u][k] >> 16)));
      }
      *reinterpret_cast<u32x4_t*>(&sh.xs[row][8 * q]) = h;
    }
  }
  __syncthreads();
  if (a.has_res && threadIdx.x == 0) add_agent(sy(a, kSyLoaded + gb % kNormCopies), 1u);
  // the rows' rstd: lane r of the first wave polls word r of line gb % kNormCopies
  if (threadIdx.x < 64) {
    const int l = threadIdx.x;
    const float* line = reinterpret_cast<const float*>(sy(a, kSyRstd + gb % kNormCopies));
    float v = 1.0f;
    int it = 0;
    while (true) {
      if (l < a.R) v = ld_agent(line + l);
      if (__all(v != 0.0f)) break;
      __builtin_amdgcn_s_sleep(4);
      if (++it > a.spin) {
        if (l == 0) __hip_atomic_fetch_or(sy(a, kSyError), kErrNormWait, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
    }
    if (l < a.R) sh.red[0][l] = v;
  }
  __syncthreads();
  TRACE_POINT(1);
#pragma unroll
  for (int u = 0; u < kXnChunks; ++u) {
    const int row = r0 + u * rpp;
    if (on && row < a.R) {
      const float rstd = sh.red[0][row];
      u32x4_t* p = reinterpret_cast<u32x4_t*>(&sh.xs[row][8 * q]);
      const u32x4_t h = *p;
      u32x4_t o;
#pragma unroll
      for (int k = 0; k < 4; ++k)
        o[k] = f2bf2(bf2f((uint16_t)h[k]) * rstd * (1.0f + bf2f((uint16_t)in.w[k])),
                     bf2f((uint16_t)(h[k] >> 16)) * rstd * (1.0f + bf2f((uint16_t)(in.w[k] >> 16))));
      *p = o;
    }
  }
  __syncthreads();
}

// MXFP4: wave w takes the (row, 512-wide unit) pairs w, w + 4, ...; lane l the chunk
// unit * 64 + l of the pair's row, so a wave's 64 chunks are one unit (the quantiser's
// layout: 4 lanes per 32-block, 16 blocks per unit)
constexpr int kXqPairs = GDN_MAX_ROWS * kKr / 512 / 4;  // pairs per wave at most
__device__ __forceinline__ void xqin_issue(const Args& a, int k0, XnIn& in) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, nu = a.Kr >> 9;
#pragma unroll
  for (int i = 0; i < kXqPairs; ++i) {
    const int pr = wave + 4 * i, row = pr / nu, unit = pr - row * nu;
    if (pr < a.R * nu)
      in.v[i] = *reinterpret_cast<const u32x4_t*>(a.x + (size_t)row * a.H + k0 + 512 * unit + 8 * lane);
  }
}
__device__ __forceinline__ void xqin_store(const Args& a, const XnIn& in, ProjShared& sh) {
  uint8_t* lds = reinterpret_cast<uint8_t*>(&sh.xs[0][0]);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, kb = (lane >> 2) & 3;
  const int nu = a.Kr >> 9, spr = a.Kr >> 7;
#pragma unroll
  for (int i = 0; i < kXqPairs; ++i) {
    const int pr = wave + 4 * i, row = pr / nu, unit = pr - row * nu;
    if (pr < a.R * nu) {  // uniform over the wave
      const uint32_t v[4] = {in.v[i][0], in.v[i][1], in.v[i][2], in.v[i][3]};
      uint32_t eb;
      *reinterpret_cast<uint32_t*>(lds + row * kMxRow + 4 * (unit * 64 + lane)) = mx_quant8(v, eb, a.mx_ceil);
      // block 4 st + kb of the unit is K quarter kb of step st: one dword per quarter, byte st
      uint32_t d = 0;
#pragma unroll
      for (int st = 0; st < 4; ++st) d |= (uint32_t)__shfl((int)eb, 16 * st + 4 * kb, 64) << (8 * st);
      if (lane < 16 && (lane & 3) == 0)
        *reinterpret_cast<uint32_t*>(lds + kMxScBase + 4 * (row * (spr + 1) + 4 * unit + kb)) = d;
    }
  }
  __syncthreads();
  TRACE_POINT(1);
}

// bf16 tiles over the K range [s Kr, (s+1) Kr): with TILES, wave w streams tile t0 + w over
// the whole range; otherwise the 4 waves stream tile t0, a quarter of the range each
template <bool PACKED, bool TILES, bool RS>
__device__ void proj_bf16(const Args& a, int gb, int t0, int s, ProjShared& sh) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t = TILES ? t0 + wave : t0;
  const int nsteps = TILES ? a.Kr >> 5 : a.Kr >> 7;
  const int l0 = TILES ? 0 : wave * nsteps;  // first local K step (32 wide) of this wave
  // The 4 in_proj_qkvz tile waves of a workgroup step through their K range together, so
  // that at each step they read 4 adjacent blocks of the grouped tiled copy (see wptr;
  // measured faster than starting each wave at its own point of the range). The in_proj_ba
  // waves each start at their own point, so that the waves streaming at the same moment
  // spread over the HBM channels (a function of the tile and split only).
  const int rot = TILES ? 0 : (t * 7 + s * 3 + wave) % nsteps;
  auto lstep = [&](int i) { return l0 + (i + rot < nsteps ? i + rot : i + rot - nsteps); };

  XnIn xi;
  HIn hi;
  if (a.normed)
    xin_issue(a, s * a.Kr, xi);
  else if (RS)
    hin_issue(a, s * a.Kr, hi);
  // weight window: step i lives in register set i % kWin until consumed
  u32x4_t w[kWin];
#pragma unroll
  for (int u = 0; u < kWin; ++u)
    if (u < nsteps) w[u] = __builtin_nontemporal_load(wptr<PACKED>(a, t, s, lstep(u), lane));
  // The last P steps of the range go straight into LDS now, so that they stream during the
  // wait for the activations (the register window holds only kWin steps: deeper register
  // windows cost occupancy, measured) and the stream left after the wait is P steps shorter.
  const int P = TILES && a.wlds && nsteps >= kWin + 2 * kLdsSteps ? kLdsSteps : 0;
  const int nreg = nsteps - P;  // steps through the register window
#pragma unroll
  for (int p = 0; p < kLdsSteps; ++p)
    if (p < P)
      __builtin_amdgcn_global_load_lds((__attribute__((address_space(1))) const void*)wptr<PACKED>(a, t, s, lstep(nreg + p), lane),
                                       (__attribute__((address_space(3))) void*)&sh.wl[wave][p][0], 16, 0, 0);

  if (a.normed)
    xin_store(a, xi, sh);
  else if (RS)
    stage_h(a, gb, hi, sh);
  else
    stage_xn(a, gb, s * a.Kr, sh);
  const int xrow = min(lane & 15, a.R - 1);  // decode rows past R are clamped; never stored
  auto xload = [&](int i) {
    return *reinterpret_cast<const u32x4_t*>(&sh.xs[xrow][32 * lstep(i) + 8 * (lane >> 4)]);
  };
  f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int i0 = 0; i0 < nreg; i0 += kWin) {
#pragma unroll
    for (int u = 0; u < kWin; ++u) {
      const int i = i0 + u;
      if (i < nreg) {
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(w[u]), as_bf16x8(xload(i)), acc, 0, 0, 0);
        if (i + kWin < nreg) w[u] = __builtin_nontemporal_load(wptr<PACKED>(a, t, s, lstep(i + kWin), lane));
      }
    }
  }
  if (P) {
    wait_stores();  // vmcnt(0): the wave's LDS fills have landed (issued before every refill above)
#pragma unroll
    for (int p = 0; p < kLdsSteps; ++p)
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(sh.wl[wave][p][lane]), as_bf16x8(xload(nreg + p)), acc, 0,
                                                    0, 0);
  }
  TRACE_POINT(2);
  if (TILES)
    publish_tiles(a, t0, s, acc);
  else
    publish_reduced(a, t0, s, acc, sh.red);
  TRACE_POINT(3);
  TRACE_HWID(15);
}

// MXFP4 tiles work in units of 4 K steps of 128 (512 K): one weight-scale dword and one
// activation-scale dword per lane cover a unit, byte `st` serving step st of the unit.
constexpr int kWinMx = kKr / 512;  // units of a wave's K range, all kept in flight

struct MxUnit {
  u32x4_t c[4];  // codes of the unit's 4 steps: 32 e2m1 values of this lane's row and K quarter
  uint32_t sc;   // the 4 steps' scales of this lane's row and K quarter
};

// Block b (1 KiB of codes, or 256 B of scales) of tile t in the tiled MXFP4 / MXFP6 copies,
// grouped like the bf16 tiles (see wptr): [K range][group of 4 tiles][block of the range]
// [tile of the group], with nb blocks per K range.
__device__ __forceinline__ size_t mx_block(const Args& a, int t, int b, int nb) {
  const int s = b / nb, bb = b - s * nb;
  return (((size_t)s * (a.Tq >> 2) + (t >> 2)) * nb + bb) * 4 + (t & 3);
}

template <bool PACKED>
__device__ __forceinline__ void mx_wload(const Args& a, int t, int U, int lane, MxUnit& m) {
  const int kb = lane >> 4;
  if (PACKED) {
    const int ns = a.Kr >> 7;  // 128-wide steps per K range
#pragma unroll
    for (int st = 0; st < 4; ++st)
      m.c[st] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(
          reinterpret_cast<const uint8_t*>(a.wpk) + (mx_block(a, t, 4 * U + st, ns) * 64 + lane) * 16));
    m.sc = __builtin_nontemporal_load(a.wpk_sc + mx_block(a, t, U, a.Kr >> 9) * 64 + lane);
  } else {
    const int row = t * 16 + (lane & 15);
    const uint8_t* c = a.wqc + (size_t)row * (a.H >> 1) + 256 * U + 16 * kb;
#pragma unroll
    for (int st = 0; st < 4; ++st)
      m.c[st] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(c + 64 * st));
    // the unit's 16 scale bytes of this row: byte 4 st + kb is step st, quarter kb
    const u32x4_t q = *reinterpret_cast<const u32x4_t*>(a.wqs + (size_t)row * (a.H >> 5) + 16 * U);
    m.sc = ((q[0] >> (8 * kb)) & 0xffu) | (((q[1] >> (8 * kb)) & 0xffu) << 8) |
           (((q[2] >> (8 * kb)) & 0xffu) << 16) | (((q[3] >> (8 * kb)) & 0xffu) << 24);
  }
}

// waits for the norm rows, then copies the MXFP4 image of xn[0..R)[k0, k0 + Kr) into LDS:
// codes at row * kMxRow, scale dwords (grouped per unit as in the global image) after them
__device__ __forceinline__ void stage_xq(const Args& a, int gb, int k0, ProjShared& sh) {
  wait_count(sy(a, kSyNorm + gb % kNormCopies), (uint32_t)(a.R * a.P), sy(a, kSyError), kErrNormWait, a.spin);
  TRACE_POINT(1);
  uint8_t* lds = reinterpret_cast<uint8_t*>(&sh.xs[0][0]);
  // 16-byte code chunks: cpr per row (<= 32), rpp >= 8 rows per pass; scale dwords: spr per
  // row (<= 8), all rows in one pass
  const int cpr = a.Kr >> 5, rpp = kThreads / cpr, r0 = threadIdx.x / cpr, q = threadIdx.x - r0 * cpr;
  const int spr = a.Kr >> 7, rs = threadIdx.x / spr, qs = threadIdx.x - rs * spr;
  constexpr int kPass = GDN_MAX_ROWS / 8;
  u32x4_t v[kPass];
  uint32_t sv = 0;
#pragma unroll
  for (int u = 0; u < kPass; ++u) {
    const int row = r0 + u * rpp;
    if (row < a.R)
      v[u] = *reinterpret_cast<const u32x4_t*>(reinterpret_cast<const uint8_t*>(a.xq) + (size_t)row * (a.H >> 1) +
                                               (k0 >> 1) + 16 * q);
  }
  if (rs < a.R) sv = a.xqs[(size_t)rs * (a.H >> 7) + (k0 >> 7) + qs];
#pragma unroll
  for (int u = 0; u < kPass; ++u) {
    const int row = r0 + u * rpp;
    if (row < a.R) *reinterpret_cast<u32x4_t*>(lds + row * kMxRow + 16 * q) = v[u];
  }
  if (rs < a.R) *reinterpret_cast<uint32_t*>(lds + kMxScBase + 4 * (rs * (spr + 1) + qs)) = sv;
  __syncthreads();
}

template <int ST>
__device__ __forceinline__ f32x4_t mx_mfma(const MxUnit& w, const u32x4_t x, uint32_t xs, f32x4_t acc) {
  const i32x8_t A = {(int)w.c[ST][0], (int)w.c[ST][1], (int)w.c[ST][2], (int)w.c[ST][3], 0, 0, 0, 0};
  const i32x8_t B = {(int)x[0], (int)x[1], (int)x[2], (int)x[3], 0, 0, 0, 0};
  // formats 4 = e2m1 for both operands; op_sel picks scale byte ST of each scale dword
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A, B, acc, 4, 4, ST, (int)w.sc, ST, (int)xs);
}

// MXFP4 in_proj_qkvz: wave w streams tile t0 + w over the K range [s Kr, (s+1) Kr)
template <bool PACKED>
__device__ void proj_mx(const Args& a, int gb, int t0, int s, ProjShared& sh) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, kb = lane >> 4;
  const int t = t0 + wave;
  const int nu = a.Kr >> 9, u0 = s * nu;  // units in the range; first global unit
  const int rot = (t * 7 + s * 3) % nu;   // spread concurrent streams over the channels
  auto lunit = [&](int m) { return m + rot < nu ? m + rot : m + rot - nu; };
  XnIn xi;
  const bool own = a.normed && a.P == 0;  // quantise the K range here (a normed input at <= 2 rows)
  if (own) xqin_issue(a, s * a.Kr, xi);
  MxUnit w[kWinMx];
#pragma unroll
  for (int m = 0; m < kWinMx; ++m)
    if (m < nu) mx_wload<PACKED>(a, t, u0 + lunit(m), lane, w[m]);

  if (own)
    xqin_store(a, xi, sh);
  else
    stage_xq(a, gb, s * a.Kr, sh);
  const int xrow = min(lane & 15, a.R - 1);  // decode rows past R are clamped; never stored
  const uint8_t* lds = reinterpret_cast<const uint8_t*>(&sh.xs[0][0]);
  const uint8_t* xc = lds + xrow * kMxRow + 16 * kb;
  const uint32_t* xsc = reinterpret_cast<const uint32_t*>(lds + kMxScBase) + xrow * ((a.Kr >> 7) + 1) + kb;
  f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int m = 0; m < kWinMx; ++m) {
    if (m < nu) {
      const int ul = lunit(m);
      const uint32_t xs = xsc[4 * ul];
      acc = mx_mfma<0>(w[m], *reinterpret_cast<const u32x4_t*>(xc + 256 * ul), xs, acc);
      acc = mx_mfma<1>(w[m], *reinterpret_cast<const u32x4_t*>(xc + 256 * ul + 64), xs, acc);
      acc = mx_mfma<2>(w[m], *reinterpret_cast<const u32x4_t*>(xc + 256 * ul + 128), xs, acc);
      acc = mx_mfma<3>(w[m], *reinterpret_cast<const u32x4_t*>(xc + 256 * ul + 192), xs, acc);
    }
  }
  TRACE_POINT(2);
  publish_tiles(a, t0, s, acc);
  TRACE_POINT(3);
  TRACE_HWID(15);
}

// MXFP6 E2M3 in_proj_qkvz with bf16 activations (W6A16, "vLLM PR #60833", a reviewer's
// comment proposing MXFP6 for the GDN projections: one v_cvt_scalef32_pk32_bf16_fp6 turns
// a lane's 32 codes times their block scale into 32 bf16 values exactly, and those feed
// the bf16 matrix cores with the bf16 activations). In a unit of 128 K, lane l holds the
// 32 codes of row l % 16 at k = 128 U + 32 (l / 16) (24 bytes, one e8m0 scale); converted,
// its 4 runs of 8 bf16 are the A operands of 4 MFMAs whose B operands are the activations
// at k = 128 U + 32 (l / 16) + 8 i, so within a unit the K order differs from the bf16
// tiles' in the same way for both operands. A wave streams tile t0 + wave over the K
// range in groups of 4 units (one scale dword per lane and group) and keeps every group
// of the range in flight.
constexpr int kGrp6 = kKr / 512;  // groups of 4 units in a K range at most

struct Mx6Group {
  u32x4_t lo[4];  // the first 16 code bytes of each unit
  u32x2_t hi[4];  // the last 8
  uint32_t sc;    // byte u: the scale of unit u
};

template <bool PACKED>
__device__ __forceinline__ void mx6_wload(const Args& a, int t, int G, int lane, Mx6Group& m) {
  if (PACKED) {
    // a unit is 1.5 KiB: the 64 lanes' 16-byte parts, then their 8-byte parts
    const int nu = a.Kr >> 7;  // units per K range
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const uint8_t* u0 = reinterpret_cast<const uint8_t*>(a.wpk) + mx_block(a, t, 4 * G + u, nu) * 1536;
      m.lo[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(u0 + 16 * lane));
      m.hi[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(u0 + 1024 + 8 * lane));
    }
    m.sc = __builtin_nontemporal_load(a.wpk_sc + mx_block(a, t, G, a.Kr >> 9) * 64 + lane);
  } else {
    // row-major codes [Nq, H/32, 24]: block 16 G + 4 u + kb of the row is unit u's
    const int row = t * 16 + (lane & 15), kb = lane >> 4;
    const uint8_t* c = a.wqc + ((size_t)row * (a.H >> 5) + 16 * G + kb) * 24;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const u32x2_t p0 = *reinterpret_cast<const u32x2_t*>(c + 96 * u);
      const u32x2_t p1 = *reinterpret_cast<const u32x2_t*>(c + 96 * u + 8);
      m.lo[u] = u32x4_t{p0[0], p0[1], p1[0], p1[1]};
      m.hi[u] = *reinterpret_cast<const u32x2_t*>(c + 96 * u + 16);
    }
    const u32x4_t q = *reinterpret_cast<const u32x4_t*>(a.wqs + (size_t)row * (a.H >> 5) + 16 * G);
    m.sc = ((q[0] >> (8 * kb)) & 0xffu) | (((q[1] >> (8 * kb)) & 0xffu) << 8) |
           (((q[2] >> (8 * kb)) & 0xffu) << 16) | (((q[3] >> (8 * kb)) & 0xffu) << 24);
  }
}

template <bool PACKED>
__device__ void proj_mx6(const Args& a, int gb, int t0, int s, ProjShared& sh) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, kb = lane >> 4;
  const int t = t0 + wave;
  const int ng = a.Kr >> 9, g0 = s * ng;  // groups in the range; first global group
  const int rot = (t * 7 + s * 3) % ng;   // spread concurrent streams over the channels
  auto lgrp = [&](int m) { return m + rot < ng ? m + rot : m + rot - ng; };
  XnIn xi;
  HIn hi;
  if (a.normed)
    xin_issue(a, s * a.Kr, xi);
  else
    hin_issue(a, s * a.Kr, hi);
  Mx6Group w[kGrp6];
#pragma unroll
  for (int m = 0; m < kGrp6; ++m)
    if (m < ng) mx6_wload<PACKED>(a, t, g0 + lgrp(m), lane, w[m]);

  if (a.normed)
    xin_store(a, xi, sh);
  else
    stage_h(a, gb, hi, sh);
  const int xrow = min(lane & 15, a.R - 1);  // decode rows past R are clamped; never stored
  f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int m = 0; m < kGrp6; ++m) {
    if (m < ng) {
      const int gl = lgrp(m);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        // the scale operand's exponent field is the e8m0 byte: the conversion multiplies by
        // 2^(byte - 127) exactly
        const float scale = __uint_as_float(((w[m].sc >> (8 * u)) & 0xffu) << 23);
        const u32x6_t src = {w[m].lo[u][0], w[m].lo[u][1], w[m].lo[u][2], w[m].lo[u][3], w[m].hi[u][0], w[m].hi[u][1]};
        const bf16x32_t v = __builtin_amdgcn_cvt_scalef32_pk32_bf16_fp6(src, scale);
        const uint16_t* xk = &sh.xs[xrow][128 * (4 * gl + u) + 32 * kb];
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_shufflevector(v, v, 0, 1, 2, 3, 4, 5, 6, 7),
                                                      as_bf16x8(*reinterpret_cast<const u32x4_t*>(xk)), acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_shufflevector(v, v, 8, 9, 10, 11, 12, 13, 14, 15),
                                                      as_bf16x8(*reinterpret_cast<const u32x4_t*>(xk + 8)), acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            __builtin_shufflevector(v, v, 16, 17, 18, 19, 20, 21, 22, 23),
            as_bf16x8(*reinterpret_cast<const u32x4_t*>(xk + 16)), acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            __builtin_shufflevector(v, v, 24, 25, 26, 27, 28, 29, 30, 31),
            as_bf16x8(*reinterpret_cast<const u32x4_t*>(xk + 24)), acc, 0, 0, 0);
      }
    }
  }
  TRACE_POINT(2);
  publish_tiles(a, t0, s, acc);
  TRACE_POINT(3);
  TRACE_HWID(15);
}

// projection workgroup gb: groups of 4 in_proj_qkvz tiles first, then the b|a tiles; S K
// ranges each
template <bool PACKED, int FMT>
__device__ void proj_role(const Args& a, int gb, ProjShared& sh) {
  // With MXFP4 weights (13.4 MB at the TP8-rank shape) the launch is bound by the norm
  // hand-off rather than by the weight stream: holding the projection workgroups' first
  // weight loads back by ~0.3 us lets the norm rows' loads through first. Measured at the
  // TP8-rank shape: 0.35-0.5 us faster at 1-8 rows, 0.05-0.1 us slower at 12-16 rows; with
  // bf16 or MXFP6 weights any delay costs time (the stream is the critical path there).
  if (FMT == kFmtMx4 && a.P > 0 && a.R <= 8) __builtin_amdgcn_s_sleep(10);
  if (gb < a.Gq) {
    const int tg = gb / a.S, s = gb - tg * a.S;
    if (FMT == kFmtMx4)
      proj_mx<PACKED>(a, gb, 4 * tg, s, sh);
    else if (FMT == kFmtMx6)
      proj_mx6<PACKED>(a, gb, 4 * tg, s, sh);
    else
      proj_bf16<PACKED, true, true>(a, gb, 4 * tg, s, sh);
  } else {
    const int g = gb - a.Gq, tb = g / a.S, s = g - tb * a.S;
    proj_bf16<PACKED, false, FMT != kFmtMx4>(a, gb, a.Tq + tb, s, sh);
  }
}

// ---------------------------------------------------------------------------------------
// role 3: projection sums, conv, L2 norms, gates, gated delta rule and gated RMSNorm of
// one (row, value head)

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
    q.x = f2bf2(v[0], v[1]);
    q.y = f2bf2(v[2], v[3]);
    *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(base) + off) = q;
  }
};

struct RecShared {
  float y[GDN_MAX_ROWS][4][128];             // per token: projection outputs q, k, v, z of the head (bf16
                                             // values); a decode step uses token 0 only
  float gt[GDN_MAX_ROWS][2];                 // verify: per token beta and exp(g)
  int dst[GDN_MAX_ROWS];                     // verify: per token the slot its state goes to
  float qs[128], ks[128], vs[128];           // conv outputs q, k, v (SiLU, bf16 values)
  float scal[4];                             // [2] exp(g), [3] beta
  float bsum[4];
};

// one conv channel: the three previous raw inputs and the four taps, loaded ahead
struct ConvIn {
  uint16_t prev[kConvW - 1];
  uint16_t w[kConvW];
  int cc;
};

__device__ __forceinline__ void conv_load(const Args& a, int slot, int cc, ConvIn& c) {
  c.cc = cc;
  const uint16_t* st = a.conv_state + (size_t)slot * (kConvW - 1) * a.Cd + cc;
#pragma unroll
  for (int j = 0; j < kConvW - 1; ++j) c.prev[j] = st[(size_t)j * a.Cd];
  const uint2 w4 = *reinterpret_cast<const uint2*>(a.conv_w + (size_t)cc * kConvW);
  c.w[0] = (uint16_t)w4.x, c.w[1] = (uint16_t)(w4.x >> 16), c.w[2] = (uint16_t)w4.y, c.w[3] = (uint16_t)(w4.y >> 16);
}

// bf16(SiLU(sum_j w_j window_j)) with the newest input y (a bf16 value)
__device__ __forceinline__ float conv_out(const ConvIn& c, float y) {
  float s = 0.0f;
#pragma unroll
  for (int j = 0; j < kConvW - 1; ++j) s = fmaf(bf2f(c.w[j]), bf2f(c.prev[j]), s);
  s = fmaf(bf2f(c.w[kConvW - 1]), y, s);
  return rbf(silu(s));
}

// roll the channel's conv state: drop the oldest input, append y
__device__ __forceinline__ void conv_store(const Args& a, int slot, const ConvIn& c, float y) {
  uint16_t* st = a.conv_state + (size_t)slot * (kConvW - 1) * a.Cd + c.cc;
#pragma unroll
  for (int j = 0; j < kConvW - 2; ++j) st[(size_t)j * a.Cd] = c.prev[j + 1];
  st[(size_t)(kConvW - 2) * a.Cd] = f2bf(y);
}

// The split partials live split-major ([S, R, PW]), so a projection workgroup stores them
// with 16-byte stores. A reader takes 4 adjacent channels of row n per 16-byte load, S
// loads in one straight sequence (split indices past S repeat the last one, so the
// compiler issues them back to back), and adds them in split order. Plain (cached) loads
// are safe because no 128-byte line holds partials of two hand-offs: a row of PW floats
// is whole lines, each key-head group's channels are whole lines (a group is a multiple
// of 64 channels) and so is the b|a block after them (padded to 32 channels). A line is
// therefore first read only after every workgroup that writes it has been counted, so no
// cache (a CU's, or an XCD's L2) can hold a copy older than its data; caches start each
// launch clean.
constexpr int kMaxSplits = 16;
template <int N>
__device__ __forceinline__ f32x4_t sum_splits4(const f32x4_t* base, size_t stride, int S) {
  f32x4_t p[N];
#pragma unroll
  for (int q = 0; q < N; ++q) p[q] = base[(size_t)min(q, S - 1) * stride];
  f32x4_t v = p[0];
#pragma unroll
  for (int q = 1; q < N; ++q)
    if (q < S) v += p[q];
  return v;
}
template <int N>
__device__ __forceinline__ float sum_splits1(const float* base, size_t stride, int S) {
  float p[N];
#pragma unroll
  for (int q = 0; q < N; ++q) p[q] = base[(size_t)min(q, S - 1) * stride];
  float v = p[0];
#pragma unroll
  for (int q = 1; q < N; ++q)
    if (q < S) v += p[q];
  return v;
}
// projection outputs (bf16 values) of channels ch .. ch + 3 of row n (ch a multiple of 4)
__device__ __forceinline__ f32x4_t proj_quad(const Args& a, int n, int ch) {
  const size_t nn = (size_t)a.PW;
  const f32x4_t* base = reinterpret_cast<const f32x4_t*>(a.part + (size_t)n * nn + ch);
  const size_t stride = a.R * nn / 4;
  f32x4_t v = a.S <= 4 ? sum_splits4<4>(base, stride, a.S)
            : a.S <= 8 ? sum_splits4<8>(base, stride, a.S) : sum_splits4<16>(base, stride, a.S);
#pragma unroll
  for (int c = 0; c < 4; ++c) v[c] = rbf(v[c]);
  return v;
}
// projection output (a bf16 value) of channel ch of row n
__device__ __forceinline__ float proj_one(const Args& a, int n, int ch) {
  const size_t nn = (size_t)a.PW;
  const float* base = a.part + (size_t)n * nn + ch;
  const size_t stride = a.R * nn;
  return rbf(a.S <= 4 ? sum_splits1<4>(base, stride, a.S)
             : a.S <= 8 ? sum_splits1<8>(base, stride, a.S) : sum_splits1<16>(base, stride, a.S));
}

// conv channel state after the token y: drop the oldest input, append y
__device__ __forceinline__ void conv_roll(ConvIn& c, float y) {
#pragma unroll
  for (int j = 0; j < kConvW - 2; ++j) c.prev[j] = c.prev[j + 1];
  c.prev[kConvW - 2] = f2bf(y);
}

// The last recurrence workgroup past its waits clears the counters for the next launch
// (its third wave, which holds the exit ticket in lane 0): by then every projection tile
// has been counted (each group and the b|a tiles had a waiter), so every projection
// workgroup is past its norm (or rstd) wait, and no recurrence workgroup reads a counter
// again (the q|k conv counter is cleared by its owner).
__device__ __forceinline__ void rec_clear(const Args& a, uint32_t exit_ticket) {
  const int tid = threadIdx.x;
  if ((tid >> 6) == 2 && __shfl((int)exit_ticket, 0, 64) == a.Rs * a.nv - 1) {
    const int l = tid & 63;
    if (l == 0) {  // the norm workgroups may still be rewriting residual rows (past their last wait)
      int it = 0;
      while (ld_agent(sy(a, kSyNormExit)) < (uint32_t)(a.R * a.P) && ++it <= a.spin) __builtin_amdgcn_s_sleep(4);
      if (it > a.spin) __hip_atomic_fetch_or(sy(a, kSyError), kErrNormWait, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    if (l < kNormCopies) {
      st_agent(sy(a, kSyNorm + l), 0u);
      st_agent(sy(a, kSyLoaded + l), 0u);
      for (int r = 0; r < a.R; ++r) st_agent(sy(a, kSyRstd + l) + r, 0u);
    }
    for (int i = l; i < a.nk * kGroupCopies; i += 64) st_agent(sy(a, kSyGroup0 + i), 0u);
    if (l == 0) {
      st_agent(sy(a, kSyNormExit), 0u);
      st_agent(sy(a, kSyBa), 0u);
      st_agent(sy(a, kSyExit), 0u);
    }
  }
}

// One workgroup per (sequence, value head). A decode step is a sequence of one token
// whose state goes back to its own slot; a verify step runs the sequence's Tk tokens one
// after the other from its source slot, keeping the state in registers, and stores the
// state (and conv window) after token t into the slot dst[t] when that is a valid slot,
// so a caller can continue from any accepted token (the follow-up the pages leave open:
// "sgl-amd-mono PR #89", Modifications, and "vLLM PR #60833", Limitations: K1 keeps no
// state per draft token, so a rejected draft could not roll back). MULTI instantiates the
// token loop; without it the loop runs once and compiles to the single-token code (the
// loop-carried state tile costs registers the decode launches should not pay for). DST: a
// single-token verify step, whose state goes to its destination slot (decode instantiations
// never read the destination array: measured, even an untaken read of it costs them time).
template <int DK, typename ST, bool MULTI, bool DST = false>
__device__ void rec_role(const Args& a, int rb, RecShared& sh) {
  constexpr int DV = DK;
  // State tile layout: wave w owns the columns [w DV/4, (w+1) DV/4) as QW quads of 4
  // columns; its 64 lanes are QW quads x NRG row groups, lane = rg * QW + quad, and a lane
  // holds rows rg RPT + m (m < RPT) of its 4 columns (contiguous, so its k and q values are
  // a few 16-byte LDS reads). Sums over the key dim (S^T k, S^T q) then stay inside a wave:
  // an xor butterfly over the row-group bits of the lane id.
  constexpr int QW = DV / 16;          // column quads per wave
  constexpr int NRG = 64 / QW;         // row groups per wave
  constexpr int RPT = DK / NRG;        // state rows per lane
  static_assert(QW * NRG == 64 && RPT * NRG == DK && RPT >= 1 && DK <= 128, "tile shape");
  const int seq = rb / a.nv, h = rb - seq * a.nv, tid = threadIdx.x;
  const int Tk = MULTI ? a.Tk : 1;
  const int kap = h / a.r, hh = h - kap * a.r;
  const bool qk_owner = hh == a.r - 1;  // writes the key head's q|k conv state
  const int slot = a.idx[seq];
  const bool valid = slot > 0 && slot < a.slots;
  const int slot1 = DST ? a.dst[seq] : slot;  // where a single token's state goes
  const int lane = tid & 63, rg = lane / QW, cq = (tid >> 6) * QW + lane % QW;
  const size_t tile = ((size_t)a.nv * DK) * DV;  // state elements per slot
  const size_t hoff = ((size_t)h * DK) * DV + 4 * cq;

  // everything that does not depend on this launch's projections is loaded first
  float S[RPT][4];
  ConvIn c0, c1;  // threads < DK: q and k channel; threads 128.. 128+DV: v channel (c0)
  const bool qk_thread = tid < DK, v_thread = tid >= 128 && tid < 128 + DV;
  if (valid) {
#pragma unroll
    for (int m = 0; m < RPT; ++m) StateIO<ST>::load(a.ssm, slot * tile + hoff + (size_t)(rg * RPT + m) * DV, S[m]);
    if (qk_thread) {
      conv_load(a, slot, kap * DK + tid, c0);
      conv_load(a, slot, a.nk * DK + kap * DK + tid, c1);
    } else if (v_thread) {
      conv_load(a, slot, 2 * a.nk * DK + h * DV + (tid - 128), c0);
    }
  }
  const float alog = a.A_log[h], dtb = bf2f(a.dt_bias[h]);
  const uint2 gw4 = *reinterpret_cast<const uint2*>(a.gnw + 4 * cq);  // gated-norm weights of the 4 columns
  if (valid && !qk_owner) {
    // the old q|k conv rows are in registers: let the owner overwrite them
    wait_stores();
    __syncthreads();
    if (tid == 0) add_agent(sy(a, sy_conv(a, seq, kap)), 1u);
  }

  // every recurrence workgroup waits, pad rows included (see the counter clearing below)
  wait_group(a, kap);
  wait_count(sy(a, kSyBa), (uint32_t)(a.Tb * a.S), sy(a, kSyError), kErrGroupWait, a.spin);
  TRACE_POINT(1);

  uint32_t exit_ticket = 0;
  if (valid) {
    const int gbase = kap * a.GW;
    if (qk_owner && a.r > 1)  // the key head's other value heads have read the old q|k conv rows
      wait_count(sy(a, sy_conv(a, seq, kap)), (uint32_t)(a.r - 1), sy(a, kSyError), kErrConvWait, a.spin);
    // q | k | v | z channel of quad j (a multiple of 4) in block blk of the head's group
    auto qch = [&](int blk, int j) {
      return gbase + (blk == 0 ? j : blk == 1 ? DK + j : blk == 2 ? 2 * DK + hh * DV + j
                                                      : 2 * DK + a.r * DV + hh * DV + j);
    };
    TRACE_POINT(13);
    if constexpr (MULTI) {
      // every token's projection outputs and gates first, 256 / DK tokens per pass, so the
      // token loop below reads them from LDS instead of waiting for a load per token
      constexpr int kTpp = kThreads / DK;
#pragma unroll 1
      for (int t0 = 0; t0 < Tk; t0 += kTpp) {
        const int t = t0 + tid / DK, q = tid % DK;
        if (t < Tk) {
          const int blk = q / (DK / 4), j = 4 * (q % (DK / 4));
          *reinterpret_cast<f32x4_t*>(&sh.y[t][blk][j]) = proj_quad(a, seq * Tk + t, qch(blk, j));
        }
      }
      if (tid < 2 * Tk) {  // even threads b, odd threads a of token tid / 2
        const int t = tid >> 1;
        const float yg = proj_one(a, seq * Tk + t, a.Nq + kap * 2 * a.r + ((tid & 1) ? a.r : 0) + hh);
        if (tid & 1) {
          const float x = yg + dtb;
          const float sp = x > 20.0f ? x : __logf(1.0f + __expf(x));
          sh.gt[t][1] = __expf(-__expf(alog) * sp);
        } else {
          sh.gt[t][0] = __builtin_amdgcn_rcpf(1.0f + __expf(-yg));
        }
      }
      // the destination slots too: a load inside the token loop would wait for every store
      // of the tokens before it (a wave's memory counter returns in order)
      if (tid >= 192 && tid < 192 + Tk) sh.dst[tid - 192] = a.dst[seq * Tk + tid - 192];
      if (tid == 128) exit_ticket = add_agent(sy(a, kSyExit), 1u);
    }
    TRACE_POINT(14);
#pragma unroll 1
    for (int t = 0; t < Tk; ++t) {
      const int n = seq * Tk + t;  // the token's projection row
      if (MULTI || t > 0) __syncthreads();  // the previous token is done with the shared arrays
      const int dslot = MULTI ? sh.dst[t] : slot1;
      const bool keep = dslot > 0 && dslot < a.slots;  // store the state after this token
      if constexpr (MULTI) {
        if (tid == 0) {
          sh.scal[3] = sh.gt[t][0];
          sh.scal[2] = sh.gt[t][1];
        }
      } else {
        // threads < DK: one quad of the head's channels each, q | k | v | z in DK / 4 quads apiece
        if (tid < DK) {
          const int blk = tid / (DK / 4), j = 4 * (tid % (DK / 4));
          *reinterpret_cast<f32x4_t*>(&sh.y[0][blk][j]) = proj_quad(a, n, qch(blk, j));
        }
        // the two gates are independent chains: thread 128 takes b, thread 192 takes a
        float yg = 0.0f;
        if (tid == 128 || tid == 192) yg = proj_one(a, n, a.Nq + kap * 2 * a.r + (tid == 192 ? a.r : 0) + hh);
        // past every wait of this workgroup: count it (loads complete in issue order, so the
        // atomic goes after this wave's loads to keep its latency off their path)
        if (tid == 128) exit_ticket = add_agent(sy(a, kSyExit), 1u);
        TRACE_POINT(5);
        if (tid == 128) {
          sh.scal[3] = __builtin_amdgcn_rcpf(1.0f + __expf(-yg));  // beta = sigmoid(b)
        } else if (tid == 192) {
          const float x = yg + dtb;
          const float sp = x > 20.0f ? x : __logf(1.0f + __expf(x));
          sh.scal[2] = __expf(-__expf(alog) * sp);  // exp(g), g = -exp(A_log) softplus(a + dt_bias)
        }
      }
      TRACE_POINT(8);
      // Nothing is in flight here in a single-token step (the projection outputs, gate
      // inputs and exit ticket have all been used). Said explicitly, the conv window and
      // state registers are known ready, so the conv-window stores below are not waited for
      // before the state pass (measured: a write round trip for the whole workgroup).
      if constexpr (!MULTI) __builtin_amdgcn_s_waitcnt(kWaitVm0);
      __syncthreads();
      TRACE_POINT(9);
      const int ty = MULTI ? t : 0;
      const int j = tid - 128;
      if (qk_thread) {
        const float yq = sh.y[ty][0][tid], yk = sh.y[ty][1][tid];
        sh.qs[tid] = conv_out(c0, yq);
        sh.ks[tid] = conv_out(c1, yk);
        if (qk_owner && keep) {
          conv_store(a, dslot, c0, yq);
          conv_store(a, dslot, c1, yk);
        }
        conv_roll(c0, yq);
        conv_roll(c1, yk);
      } else if (v_thread) {
        const float yv = sh.y[ty][2][j];
        sh.vs[j] = conv_out(c0, yv);
        if (keep) conv_store(a, dslot, c0, yv);
        conv_roll(c0, yv);
      }
      __syncthreads();
      TRACE_POINT(2);
      // One pass over the old state with the raw (not yet normalised) conv outputs k and q:
      // per lane, the partial sums over its rows of S^T k and S^T q for its 4 columns and of
      // k.k, q.q and k.q; then sums over the row groups by an xor butterfly inside the wave,
      // after which every lane of a column quad holds the same totals.
      float v[11] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int m = 0; m < RPT; ++m) {
        const int i = rg * RPT + m;
        const float k = sh.ks[i], q = sh.qs[i];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          v[c] = fmaf(S[m][c], k, v[c]);
          v[4 + c] = fmaf(S[m][c], q, v[4 + c]);
        }
        v[8] = fmaf(k, k, v[8]);
        v[9] = fmaf(q, q, v[9]);
        v[10] = fmaf(k, q, v[10]);
      }
      TRACE_POINT(10);
      xor_butterfly<QW>(v);
      TRACE_POINT(6);
      // reciprocal square roots on the hardware instruction (within 1 ulp)
      constexpr float kInvSqrtDk = DK == 32 ? 0.17677669529663687f : DK == 64 ? 0.125f : 0.08838834764831845f;
      const float kscale = __builtin_amdgcn_rsqf(v[8] + a.l2eps);                 // 1 / |k|
      const float qscale = __builtin_amdgcn_rsqf(v[9] + a.l2eps) * kInvSqrtDk;    // 1 / (|q| sqrt(dk))
      const float decay = sh.scal[2], beta = sh.scal[3];
      const float kq = v[10] * kscale * qscale;  // (normalised k) . (normalised, scaled q)
      // With u = S^T k and w = S^T q of the old state, the updated state
      // S' = e^g S + k d^T, d = beta (v - e^g u), reads out o = S'^T q = e^g w + d (k . q).
      float d[4], ob[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        d[c] = beta * (sh.vs[4 * cq + c] - decay * (v[c] * kscale));
        ob[c] = rbf(fmaf(d[c], kq, decay * (v[4 + c] * qscale)));
      }
      TRACE_POINT(11);
      // RMSNormGated over the head. Every row group of a wave holds the wave's DV / 4
      // columns once: the sum of ob^2 over its QW column quads (an xor butterfly over the
      // quad bits of the lane id, fixed order), then over the 4 waves through LDS.
      float ss = (ob[0] * ob[0] + ob[1] * ob[1]) + (ob[2] * ob[2] + ob[3] * ob[3]);
      if (QW >= 2) ss += dpp<0xB1>(ss);  // xor 1
      if (QW >= 4) ss += dpp<0x4E>(ss);  // xor 2
      if (QW >= 8) ss += dpp<0x141>(ss);  // the other quad of lanes among 8 (mirror)
      if (lane == 0) sh.bsum[tid >> 6] = ss;
      // The state update and its stores overlap the exchange; with the out_proj fold they
      // follow the core row instead, whose completion is signalled before they are issued.
      auto update_state = [&]() {
#pragma unroll
        for (int m = 0; m < RPT; ++m) {
          const float kh = sh.ks[rg * RPT + m] * kscale;
#pragma unroll
          for (int c = 0; c < 4; ++c) S[m][c] = fmaf(decay, S[m][c], kh * d[c]);
          if (keep) StateIO<ST>::store(a.ssm, dslot * tile + hoff + (size_t)(rg * RPT + m) * DV, S[m]);
        }
      };
      if (!a.fold) update_state();
      TRACE_POINT(7);
      __syncthreads();
      ss = (sh.bsum[0] + sh.bsum[1]) + (sh.bsum[2] + sh.bsum[3]);
      TRACE_POINT(12);
      const float rstd = __builtin_amdgcn_rsqf(ss * (1.0f / (float)DV) + a.geps);
      if (rg == 0) {
        const float g0 = bf2f((uint16_t)gw4.x), g1 = bf2f((uint16_t)(gw4.x >> 16));
        const float g2 = bf2f((uint16_t)gw4.y), g3 = bf2f((uint16_t)(gw4.y >> 16));
        const float* z = &sh.y[ty][3][4 * cq];
        const uint64_t o = (uint64_t)f2bf2(ob[0] * rstd * g0 * silu(z[0]), ob[1] * rstd * g1 * silu(z[1])) |
                           ((uint64_t)f2bf2(ob[2] * rstd * g2 * silu(z[2]), ob[3] * rstd * g3 * silu(z[3])) << 32);
        uint64_t* dst = reinterpret_cast<uint64_t*>(a.core + (size_t)n * a.nv * DV + (size_t)h * DV + 4 * cq);
        if (a.fold)  // read by the out_proj workgroups: coherent at agent scope
          __hip_atomic_store(dst, o, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        else
          *dst = o;
      }
      if (a.fold) {  // the head's core row is in place for the out_proj workgroups (one token)
        wait_stores();
        __syncthreads();
        if (tid < kCoreCopies) add_agent(sy(a, kSyCoreDone + tid), 1u);
        update_state();
      }
      TRACE_POINT(3);
    }
    if (qk_owner && tid == 0 && a.r > 1) st_agent(sy(a, sy_conv(a, seq, kap)), 0u);
  } else {
    if (tid == 128) exit_ticket = add_agent(sy(a, kSyExit), 1u);
    // pad sequence: a zero core row for each of its tokens
    for (int t = 0; t < Tk; ++t) {
      uint16_t* core = a.core + (size_t)(seq * Tk + t) * a.nv * DV + (size_t)h * DV;
      for (int j = 2 * tid; j < DV; j += 2 * kThreads) st_agent(reinterpret_cast<uint32_t*>(core + j), 0u);
    }
  }
  if (a.fold && !valid) {  // the pad row's zero core row is in place for the out_proj workgroups
    wait_stores();
    __syncthreads();
    if (tid < kCoreCopies) add_agent(sy(a, kSyCoreDone + tid), 1u);
  }

  rec_clear(a, exit_ticket);
  TRACE_POINT(4);
}

// ---------------------------------------------------------------------------------------
// role 3, verify steps of more than one token at head dim 128: the delta rule unrolled over
// the step's tokens, so that only the elementwise state update stays serial. With k_t and
// q_t normalised (q_t also scaled by 1/sqrt(dk)), a_t = exp(g_t), Gm(i..t) the product of
// a_i .. a_t (1 when empty) and S0 the state the step starts from, substituting the update
// S_t = a_t S_{t-1} + k_t d_t^T into itself gives
//   a_t S_{t-1}^T k_t = Gm(0..t) S0^T k_t + sum_{j<t} Gm(j+1..t) (k_j . k_t) d_j
//   d_t = beta_t (v_t - a_t S_{t-1}^T k_t)
//   o_t = S_t^T q_t   = Gm(0..t) S0^T q_t + sum_{j<=t} Gm(j+1..t) (k_j . q_t) d_j
// (the recurrence the decode steps run, one token after the other, in another order of
// rounding). So: S0^T k_t and S0^T q_t for every token at once, and the key and query dot
// products, are matrix-core products (bf16 operands: the conv outputs are bf16 values, and
// so is a bf16 state; an f32 state goes in as two bf16 terms, hi + lo, which keeps about 16
// significant bits of each element); the per-token scalars and the coefficients are small
// tables in LDS; d_t and o_t follow per column, a forward substitution over the tokens;
// then the gated norm and the core rows of all tokens; and last the serial part, the state
// update and the snapshot stores, with no barrier and no wait between the tokens.
// one token's rows, padded so that consecutive tokens start 16 bytes apart in the LDS
// banks (lanes reading 16 tokens' rows at one offset, as the matrix-core operands do,
// would otherwise all hit the same banks)
struct TokRows {
  float b[4][128];  // q, k, v, z
  float pad[4];
};
constexpr int kURow = 132;  // padded row of u and w, for the same reason
struct VerShared {
  TokRows y[GDN_MAX_ROWS];        // per token: projections q, k, v, z; then q, k, v conv outputs
  float u[GDN_MAX_ROWS][kURow];   // S0^T k_t (k not normalised), then d_t
  float w[GDN_MAX_ROWS][kURow];   // S0^T q_t (q not normalised), then o_t (bf16 values)
  float kk[GDN_MAX_ROWS][GDN_MAX_ROWS + 1];  // k_t . k_j, then Gm(j+1..t) (k_j . k_t), j < t
  float qk[GDN_MAX_ROWS][GDN_MAX_ROWS + 1];  // q_t . k_j, then Gm(j+1..t) (k_j . q_t), j <= t
  float qq[GDN_MAX_ROWS];                    // q_t . q_t
  float ks[GDN_MAX_ROWS], qs[GDN_MAX_ROWS];  // 1 / |k_t|, 1 / (|q_t| sqrt(dk))
  float gc[GDN_MAX_ROWS];                    // Gm(0..t)
  float gt[GDN_MAX_ROWS][2];                 // beta_t, a_t
  float ga[GDN_MAX_ROWS];                    // a_t again, contiguous
  int dst[GDN_MAX_ROWS];                     // the slot the state after token t goes to
};

// bf16 pair of two floats that are bf16 values (exact: their low 16 bits are zero)
__device__ __forceinline__ uint32_t bf16_pair(float lo, float hi) {
  return (__builtin_bit_cast(uint32_t, lo) >> 16) | (__builtin_bit_cast(uint32_t, hi) & 0xffff0000u);
}
// bf16 image of 8 consecutive floats in LDS that are bf16 values
__device__ __forceinline__ u32x4_t bf16x8_of(const float* p) {
  const f32x4_t a = *reinterpret_cast<const f32x4_t*>(p), b = *reinterpret_cast<const f32x4_t*>(p + 4);
  return u32x4_t{bf16_pair(a[0], a[1]), bf16_pair(a[2], a[3]), bf16_pair(b[0], b[1]), bf16_pair(b[2], b[3])};
}

// (Its profiling-build timeline points are few on purpose: more of them made that build of
// the role spill registers, which distorts the timeline.)
template <typename ST>
__device__ __forceinline__ void rec_verify(const Args& a, int rb, VerShared& sh) {
  constexpr int D = 128;
  constexpr bool kF32 = sizeof(ST) == 4;
  // State tile layout: wave w holds the column half ch = w & 1 and the row half rh = w >> 1;
  // lane l holds the 4 columns 64 ch + 4 (l & 15) .. + 3 of the 16 rows 64 rh + 16 (l >> 4)
  // .. + 15. Rows m0 .. m0 + 7 of one column j are then lane l's part of a 16x16x32 bf16
  // matrix-core B operand (K index 8 (l >> 4) + i <-> row 64 rh + 16 (l >> 4) + m0 + i,
  // N index l & 15 <-> column 64 ch + 4 (l & 15) + j), and a store of row m covers 64
  // contiguous columns of 4 rows, whole 128-byte lines.
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int ch = wave & 1, rh = wave >> 1, qd = lane & 15, rg = lane >> 4;
  const int r0 = 64 * rh + 16 * rg, c0 = 64 * ch + 4 * qd;
  const int seq = rb / a.nv, h = rb - seq * a.nv, Tk = a.Tk;
  const int kap = h / a.r, hh = h - kap * a.r;
  const bool qk_owner = hh == a.r - 1;
  const int slot = a.idx[seq];
  const bool valid = slot > 0 && slot < a.slots;
  const size_t tile = ((size_t)a.nv * D) * D;
  const size_t hoff = ((size_t)h * D) * D + c0;

  // The old state: an f32 pool's rows as f32; a bf16 pool's rows kept as loaded (2 bf16
  // pairs per row, half the registers) until the serial part needs them as f32.
  float S[16][4];
  uint32_t Sb[16][2];
  ConvIn c0c, c1c;  // threads < 128: q and k channel tid; threads 128..255: v channel tid - 128
  const bool qk_thread = tid < D;
  if (valid) {
#pragma unroll
    for (int m = 0; m < 16; ++m) {
      const size_t off = slot * tile + hoff + (size_t)(r0 + m) * D;
      if constexpr (kF32) {
        StateIO<float>::load(a.ssm, off, S[m]);
      } else {
        const uint2 q = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint16_t*>(a.ssm) + off);
        Sb[m][0] = q.x, Sb[m][1] = q.y;
      }
    }
    if (qk_thread) {
      conv_load(a, slot, kap * D + tid, c0c);
      conv_load(a, slot, a.nk * D + kap * D + tid, c1c);
    } else {
      conv_load(a, slot, 2 * a.nk * D + h * D + (tid - D), c0c);
    }
  }
  const float alog = a.A_log[h], dtb = bf2f(a.dt_bias[h]);
  const int p16 = tid & 15;  // the 8 columns 8 p16 .. + 7 of the output phase
  const uint4 gw8 = *reinterpret_cast<const uint4*>(a.gnw + 8 * p16);
  if (valid && !qk_owner) {
    // the old q|k conv rows are in registers: let the owner overwrite them
    wait_stores();
    __syncthreads();
    if (tid == 0) add_agent(sy(a, sy_conv(a, seq, kap)), 1u);
  }
  wait_group(a, kap);
  wait_count(sy(a, kSyBa), (uint32_t)(a.Tb * a.S), sy(a, kSyError), kErrGroupWait, a.spin);
  TRACE_POINT(1);

  uint32_t exit_ticket = 0;
  if (!valid) {
    if (tid == 128) exit_ticket = add_agent(sy(a, kSyExit), 1u);
    for (int t = 0; t < Tk; ++t) {  // pad sequence: a zero core row for each of its tokens
      uint16_t* core = a.core + (size_t)(seq * Tk + t) * a.nv * D + (size_t)h * D;
      if (tid < D / 2) st_agent(reinterpret_cast<uint32_t*>(core) + tid, 0u);
    }
    rec_clear(a, exit_ticket);
    return;
  }
  if (qk_owner && a.r > 1)  // the key head's other value heads have read the old q|k conv rows
    wait_count(sy(a, sy_conv(a, seq, kap)), (uint32_t)(a.r - 1), sy(a, kSyError), kErrConvWait, a.spin);

  // every token's projection outputs (q | k | v | z quads of the head), 2 tokens per pass
  // and kVerPasses passes' loads in flight together (each pass holds S 16-byte loads while
  // the state tile is in registers too); the gates and the destination slots
  {
    constexpr int kVerPasses = 2;
    const int gbase = kap * a.GW, q = tid & 127, blk = q >> 5, j = 4 * (q & 31);
    const int chn = gbase + (blk == 0 ? j : blk == 1 ? D + j : blk == 2 ? 2 * D + hh * D + j
                                                      : 2 * D + a.r * D + hh * D + j);
    // the gate inputs first (even threads b, odd threads a of token tid / 2): their loads
    // then return before the threads' own token outputs, not a round trip after them
    const float yg = tid < 2 * Tk ? proj_one(a, seq * Tk + (tid >> 1), a.Nq + kap * 2 * a.r + ((tid & 1) ? a.r : 0) + hh)
                                  : 0.0f;
#pragma unroll 1
    for (int p0 = 0; p0 < Tk; p0 += 2 * kVerPasses) {
      f32x4_t v[kVerPasses];
#pragma unroll
      for (int u = 0; u < kVerPasses; ++u)
        v[u] = proj_quad(a, seq * Tk + min(p0 + 2 * u + (tid >> 7), Tk - 1), chn);
#pragma unroll
      for (int u = 0; u < kVerPasses; ++u) {
        const int t = p0 + 2 * u + (tid >> 7);
        if (t < Tk) *reinterpret_cast<f32x4_t*>(&sh.y[t].b[blk][j]) = v[u];
      }
    }
    if (tid < 2 * Tk) {
      const int t = tid >> 1;
      if (tid & 1) {
        const float x = yg + dtb;
        const float sp = x > 20.0f ? x : __logf(1.0f + __expf(x));
        sh.gt[t][1] = sh.ga[t] = __expf(-__expf(alog) * sp);  // exp(g), g = -exp(A_log) softplus(a + dt_bias)
      } else {
        sh.gt[t][0] = __builtin_amdgcn_rcpf(1.0f + __expf(-yg));  // beta = sigmoid(b)
      }
    }
    if (tid >= 192 && tid < 192 + Tk) sh.dst[tid - 192] = a.dst[seq * Tk + tid - 192];
    // past every wait of this workgroup: count it (the atomic's return is waited for at
    // once, after this wave's loads; taken at the end instead, its wait there would also
    // wait for the snapshot stores before the last workgroup clears the counters: measured)
    if (tid == 128) exit_ticket = add_agent(sy(a, kSyExit), 1u);
  }
  // Nothing is in flight here (every load above has been consumed). Saying so explicitly
  // tells the compiler that the old state's registers are ready: otherwise its first use
  // (the matrix-core operands, after the conv-window stores below) gets a wait for every
  // memory operation before it, those stores included (measured: a write round trip).
  __builtin_amdgcn_s_waitcnt(kWaitVm0);
  __syncthreads();
  TRACE_POINT(14);

  // conv of every token, one channel per thread, in token order (measured faster than
  // reading all of the channel's inputs first); the window after each kept token goes to
  // its slot
  if (qk_thread) {
#pragma unroll 1
    for (int t = 0; t < Tk; ++t) {
      const float yq = sh.y[t].b[0][tid], yk = sh.y[t].b[1][tid];
      sh.y[t].b[0][tid] = conv_out(c0c, yq);
      sh.y[t].b[1][tid] = conv_out(c1c, yk);
      const int ds = sh.dst[t];
      if (qk_owner && ds > 0 && ds < a.slots) {
        conv_store(a, ds, c0c, yq);
        conv_store(a, ds, c1c, yk);
      }
      conv_roll(c0c, yq);
      conv_roll(c1c, yk);
    }
  } else {
    const int j = tid - D;
#pragma unroll 1
    for (int t = 0; t < Tk; ++t) {
      const float yv = sh.y[t].b[2][j];
      sh.y[t].b[2][j] = conv_out(c0c, yv);
      const int ds = sh.dst[t];
      if (ds > 0 && ds < a.slots) conv_store(a, ds, c0c, yv);
      conv_roll(c0c, yv);
    }
  }
  __syncthreads();
  TRACE_POINT(2);

  const int ta = lane & 15;
  const bool tok = ta < Tk;
  const u32x4_t zero = {0u, 0u, 0u, 0u};
  // the tokens' dot products, one product per wave: k.k, q.k, q.q (16x16, tokens past Tk zero)
  if (wave < 3) {
    const int xa = wave == 0 ? 1 : 0, xb = wave == 2 ? 0 : 1;  // blocks: q 0, k 1
    f32x4_t g = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int s4 = 0; s4 < D / 32; ++s4) {
      const int k0 = 32 * s4 + 8 * rg;
      const u32x4_t va = tok ? bf16x8_of(&sh.y[ta].b[xa][k0]) : zero;
      const u32x4_t vb = tok ? bf16x8_of(&sh.y[ta].b[xb][k0]) : zero;
      g = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(va), as_bf16x8(vb), g, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {  // g[i] = row 4 (l >> 4) + i (the A token), column l & 15
      const int m = 4 * rg + i, n = ta;
      if (m < Tk && n < Tk) {
        if (wave == 0) sh.kk[m][n] = g[i];
        else if (wave == 1) sh.qk[m][n] = g[i];
        else if (m == n) sh.qq[m] = g[i];
      }
    }
  }
  // S0^T k_t and S0^T q_t over this wave's 64 rows for all tokens: A operand = token
  // (lane & 15)'s k (or q) at the same 8 rows as the B operand's K index. Lane l's results
  // hold, for token 4 (l >> 4) + i, the columns c0 .. c0 + 3 (one per j): the upper row
  // half's waves store theirs, then the lower half's add theirs to them.
  f32x4_t acc[2][4];
#pragma unroll
  for (int pr = 0; pr < 2; ++pr)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[pr][j] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int m0 = 0; m0 < 16; m0 += 8) {
    const u32x4_t ak = tok ? bf16x8_of(&sh.y[ta].b[1][r0 + m0]) : zero;
    const u32x4_t aq = tok ? bf16x8_of(&sh.y[ta].b[0][r0 + m0]) : zero;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      // column j, rows m0 .. m0 + 7: a bf16 pool's halves as they are; an f32 element as
      // hi + lo, both bf16 values
      auto hi = [&](int i) { return rbf(S[m0 + i][j]); };
      auto lo = [&](int i) { return rbf(S[m0 + i][j] - rbf(S[m0 + i][j])); };
      auto col2 = [&](int i) {  // rows m0 + i, m0 + i + 1 of column j of a bf16 pool
        const uint32_t x = Sb[m0 + i][j >> 1], y = Sb[m0 + i + 1][j >> 1];
        return (j & 1) ? (x >> 16) | (y & 0xffff0000u) : (x & 0xffffu) | (y << 16);
      };
      u32x4_t bh;
      if constexpr (kF32)
        bh = u32x4_t{bf16_pair(hi(0), hi(1)), bf16_pair(hi(2), hi(3)), bf16_pair(hi(4), hi(5)), bf16_pair(hi(6), hi(7))};
      else
        bh = u32x4_t{col2(0), col2(2), col2(4), col2(6)};
      acc[0][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(ak), as_bf16x8(bh), acc[0][j], 0, 0, 0);
      acc[1][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(aq), as_bf16x8(bh), acc[1][j], 0, 0, 0);
      if constexpr (kF32) {
        const u32x4_t bl = {bf16_pair(lo(0), lo(1)), bf16_pair(lo(2), lo(3)), bf16_pair(lo(4), lo(5)),
                            bf16_pair(lo(6), lo(7))};
        acc[0][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(ak), as_bf16x8(bl), acc[0][j], 0, 0, 0);
        acc[1][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(aq), as_bf16x8(bl), acc[1][j], 0, 0, 0);
      }
    }
  }
  if (rh == 1) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      *reinterpret_cast<f32x4_t*>(&sh.u[4 * rg + i][c0]) = f32x4_t{acc[0][0][i], acc[0][1][i], acc[0][2][i], acc[0][3][i]};
      *reinterpret_cast<f32x4_t*>(&sh.w[4 * rg + i][c0]) = f32x4_t{acc[1][0][i], acc[1][1][i], acc[1][2][i], acc[1][3][i]};
    }
  }
  __syncthreads();
  // the lower row half's waves complete the sums; in the same phase, the coefficient tables
  // (they touch other arrays)
  if (rh == 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f32x4_t* pu = reinterpret_cast<f32x4_t*>(&sh.u[4 * rg + i][c0]);
      f32x4_t* pw = reinterpret_cast<f32x4_t*>(&sh.w[4 * rg + i][c0]);
      *pu = *pu + f32x4_t{acc[0][0][i], acc[0][1][i], acc[0][2][i], acc[0][3][i]};
      *pw = *pw + f32x4_t{acc[1][0][i], acc[1][1][i], acc[1][2][i], acc[1][3][i]};
    }
  }
  {  // the coefficient tables, one (t, j) per thread
    const int t = tid >> 4, j = tid & 15;
    if (t < Tk && j < Tk) {
      // reciprocal square roots on the hardware instruction (within 1 ulp)
      const float kt = __builtin_amdgcn_rsqf(sh.kk[t][t] + a.l2eps), kj = __builtin_amdgcn_rsqf(sh.kk[j][j] + a.l2eps);
      const float qt = __builtin_amdgcn_rsqf(sh.qq[t] + a.l2eps) * 0.08838834764831845f;
      float av4[GDN_MAX_ROWS];  // the decays, read together (no LDS round trip per factor)
#pragma unroll
      for (int i4 = 0; i4 < GDN_MAX_ROWS / 4; ++i4) {
        const f32x4_t g4 = *reinterpret_cast<const f32x4_t*>(&sh.ga[4 * i4]);
        av4[4 * i4] = g4[0], av4[4 * i4 + 1] = g4[1], av4[4 * i4 + 2] = g4[2], av4[4 * i4 + 3] = g4[3];
      }
      float gm = 1.0f;
#pragma unroll
      for (int i = 1; i < GDN_MAX_ROWS; ++i)
        if (i > j && i <= t) gm *= av4[i];
      // in place: each thread rewrites its own entry only, and the diagonal of kk, which
      // the other threads read, stays (the coefficients of d_j in d_t need j < t only)
      if (j < t) sh.kk[t][j] = gm * sh.kk[t][j] * kt * kj;
      sh.qk[t][j] = j <= t ? gm * sh.qk[t][j] * qt * kj : 0.0f;
      if (j == 0) {
        sh.gc[t] = av4[0] * gm;
        sh.ks[t] = kt;
        sh.qs[t] = qt;
      }
    }
  }
  __syncthreads();

  // d_t and o_t, one column per thread: a forward substitution over the tokens
  if (tid < D) {
    const int c = tid;
    float dr[GDN_MAX_ROWS];
#pragma unroll
    for (int t = 0; t < GDN_MAX_ROWS; ++t) {
      if (t < Tk) {
        float acc = sh.gc[t] * (sh.u[t][c] * sh.ks[t]);
#pragma unroll
        for (int j = 0; j < t; ++j) acc = fmaf(sh.kk[t][j], dr[j], acc);
        dr[t] = sh.gt[t][0] * (sh.y[t].b[2][c] - acc);
        float o = sh.gc[t] * (sh.w[t][c] * sh.qs[t]);
#pragma unroll
        for (int j = 0; j <= t; ++j) o = fmaf(sh.qk[t][j], dr[j], o);
        sh.u[t][c] = dr[t];
        sh.w[t][c] = rbf(o);
      }
    }
  }
  __syncthreads();
  TRACE_POINT(11);

  // RMSNormGated and the core row of every token: 16 threads per token, 8 columns each
  {
    const int t = tid >> 4;
    if (t < Tk) {
      const f32x4_t o0 = *reinterpret_cast<const f32x4_t*>(&sh.w[t][8 * p16]);
      const f32x4_t o1 = *reinterpret_cast<const f32x4_t*>(&sh.w[t][8 * p16 + 4]);
      float ss = ((o0[0] * o0[0] + o0[1] * o0[1]) + (o0[2] * o0[2] + o0[3] * o0[3])) +
                 ((o1[0] * o1[0] + o1[1] * o1[1]) + (o1[2] * o1[2] + o1[3] * o1[3]));
      ss += dpp<0xB1>(ss);   // xor 1
      ss += dpp<0x4E>(ss);   // xor 2
      ss += dpp<0x141>(ss);  // the other quad among 8 (mirror)
      ss += dpp<0x128>(ss);  // the other 8 among 16 (rotate by 8)
      const float rstd = __builtin_amdgcn_rsqf(ss * (1.0f / (float)D) + a.geps);
      const f32x4_t z0 = *reinterpret_cast<const f32x4_t*>(&sh.y[t].b[3][8 * p16]);
      const f32x4_t z1 = *reinterpret_cast<const f32x4_t*>(&sh.y[t].b[3][8 * p16 + 4]);
      auto gated = [&](float o, float z, uint32_t g, int hi) {
        return o * rstd * bf2f((uint16_t)(hi ? g >> 16 : g)) * silu(z);
      };
      *reinterpret_cast<uint4*>(a.core + (size_t)(seq * Tk + t) * a.nv * D + (size_t)h * D + 8 * p16) =
          make_uint4(f2bf2(gated(o0[0], z0[0], gw8.x, 0), gated(o0[1], z0[1], gw8.x, 1)),
                     f2bf2(gated(o0[2], z0[2], gw8.y, 0), gated(o0[3], z0[3], gw8.y, 1)),
                     f2bf2(gated(o1[0], z1[0], gw8.z, 0), gated(o1[1], z1[1], gw8.z, 1)),
                     f2bf2(gated(o1[2], z1[2], gw8.w, 0), gated(o1[3], z1[3], gw8.w, 1)));
    }
  }
  TRACE_POINT(12);

  // the serial part: S_t = a_t S_{t-1} + k_t d_t^T, stored when the token's slot is valid
  if constexpr (!kF32) {
#pragma unroll
    for (int m = 0; m < 16; ++m) {
      S[m][0] = __builtin_bit_cast(float, Sb[m][0] << 16), S[m][1] = __builtin_bit_cast(float, Sb[m][0] & 0xffff0000u);
      S[m][2] = __builtin_bit_cast(float, Sb[m][1] << 16), S[m][3] = __builtin_bit_cast(float, Sb[m][1] & 0xffff0000u);
    }
  }
  // A token's LDS operands (its 16 key values of this lane's rows, d_t of its 4 columns,
  // a_t, 1/|k_t|, the slot) are read together, one token ahead, so the loop waits on no
  // LDS round trip; whether the snapshot is kept is one branch per token. (Measured: 8-byte
  // row stores beat 16-byte stores that need the neighbour lanes to swap halves.)
  struct TokIn {
    f32x4_t k[4], d;
    float dec, kst;
    int ds;
  };
  auto tok_load = [&](int t, TokIn& v) {
#pragma unroll
    for (int m4 = 0; m4 < 4; ++m4) v.k[m4] = *reinterpret_cast<const f32x4_t*>(&sh.y[t].b[1][r0 + 4 * m4]);
    v.d = *reinterpret_cast<const f32x4_t*>(&sh.u[t][c0]);
    v.dec = sh.gt[t][1];
    v.kst = sh.ks[t];
    v.ds = sh.dst[t];
  };
  auto update = [&](const TokIn& v) {
#pragma unroll
    for (int m = 0; m < 16; ++m) {
      const float kh = v.k[m >> 2][m & 3] * v.kst;
#pragma unroll
      for (int j = 0; j < 4; ++j) S[m][j] = fmaf(v.dec, S[m][j], kh * v.d[j]);
    }
  };
  auto snapshot = [&](int ds) {
    if (ds > 0 && ds < a.slots) {
      const size_t base = ds * tile + hoff;
#pragma unroll
      for (int m = 0; m < 16; ++m) StateIO<ST>::store(a.ssm, base + (size_t)(r0 + m) * D, S[m]);
    }
  };
  // two operand sets in turn: token t + 1's are read while token t is computed
  TokIn ta_, tb_;
  tok_load(0, ta_);
#pragma unroll 1
  for (int t = 0; t < Tk; t += 2) {
    if (t + 1 < Tk) tok_load(t + 1, tb_);
    update(ta_);
    snapshot(ta_.ds);
    if (t + 1 < Tk) {
      if (t + 2 < Tk) tok_load(t + 2, ta_);
      update(tb_);
      snapshot(tb_.ds);
    }
  }
  TRACE_POINT(3);
  if (qk_owner && tid == 0 && a.r > 1) st_agent(sy(a, sy_conv(a, seq, kap)), 0u);
  rec_clear(a, exit_ticket);
}

// ---------------------------------------------------------------------------------------
// role 4 (out_proj folded in): the rank's out_proj partial out = bf16(core W_out^T) for 4
// 16-column tiles of H, one per wave over the whole K = nv*dv (<= 1024). Each wave issues
// its whole tile (up to 32 KiB, held in registers) before waiting, so the out_proj weights
// stream while the recurrence runs; a wave's loads return in issue order, so that is all
// it has in flight when it polls. Then the core rows are staged in LDS once per workgroup
// and multiplied on the bf16 MFMA ("SGLang PR #43558", Modifications: K1 with the out_proj
// fold writes the rank's out_proj partial).
constexpr int kOutSteps = 32;  // 32-wide K steps of a tile at most (K <= 1024)
template <bool PACKED>
__device__ void oproj_role(const Args& a, int ob, ProjShared& sh) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, tid = threadIdx.x;
  const int K = a.Ko, nsteps = K >> 5, t = 4 * ob + wave;
  auto wop = [&](int j) -> const u32x4_t* {
    if (PACKED)
      return reinterpret_cast<const u32x4_t*>(a.wo_pk + (((size_t)t * nsteps + j) * 64 + lane) * 8);
    return reinterpret_cast<const u32x4_t*>(a.wo + (size_t)(t * 16 + (lane & 15)) * K + 32 * j + 8 * (lane >> 4));
  };
  u32x4_t w[kOutSteps];
#pragma unroll
  for (int u = 0; u < kOutSteps; ++u)
    if (u < nsteps) w[u] = __builtin_nontemporal_load(wop(u));

  wait_count(sy(a, kSyCoreDone + ob % kCoreCopies), (uint32_t)(a.Rs * a.nv), sy(a, kSyError), kErrGroupWait,
             a.spin);
  TRACE_POINT(1);
  // core rows [R, K] into LDS with direct-to-LDS loads, all in flight at once (plain
  // loads: first read after the count). One wave instruction fills 1 KiB of LDS, 16 bytes
  // per lane in lane order, so the image is unpadded [R][K]; to keep the B-operand reads
  // free of bank conflicts the 16-byte chunk c of row r sits at chunk c ^ (r % 16) of its
  // row (K is a multiple of 128, so the swizzle stays inside the row).
  const int cpr = K >> 3, nch = a.R * cpr;
  char* img = reinterpret_cast<char*>(&sh.xs[0][0]);
#pragma unroll
  for (int u = 0; u < GDN_MAX_ROWS * kKr / 8 / 64 / 4; ++u) {
    const int f0 = 64 * (4 * u + wave), f = f0 + lane;
    if (f0 < nch) {
      const int row = f / cpr, c = (f - row * cpr) ^ (row & 15);
      if (f < nch)
        __builtin_amdgcn_global_load_lds((__attribute__((address_space(1))) const void*)(a.core + (size_t)row * K + 8 * c),
                                         (__attribute__((address_space(3))) void*)(img + 16 * f0), 16, 0, 0);
    }
  }
  wait_stores();  // vmcnt(0): this wave's LDS writes have landed
  __syncthreads();
  const int xrow = min(lane & 15, a.R - 1);  // decode rows past R are clamped; never stored
  const char* xr = img + (size_t)xrow * K * 2;
  f32x4_t acc0 = {0.0f, 0.0f, 0.0f, 0.0f}, acc1 = acc0;
#pragma unroll
  for (int u = 0; u < kOutSteps; u += 2) {
    if (u < nsteps) {
      const int c0 = (4 * u + (lane >> 4)) ^ (xrow & 15), c1 = (4 * (u + 1) + (lane >> 4)) ^ (xrow & 15);
      acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
          as_bf16x8(w[u]), as_bf16x8(*reinterpret_cast<const u32x4_t*>(xr + 16 * c0)), acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
          as_bf16x8(w[u + 1]), as_bf16x8(*reinterpret_cast<const u32x4_t*>(xr + 16 * c1)), acc1, 0, 0, 0);
    }
  }
  const f32x4_t acc = acc0 + acc1;
  TRACE_POINT(2);
  // D layout: lane l holds output columns 4 (l / 16) + i of decode row l % 16
  const int en = lane & 15;
  if (en < a.R) {
    uint16_t* o = a.out + (size_t)en * a.H + t * 16 + 4 * (lane >> 4);
    *reinterpret_cast<uint2*>(o) = make_uint2(f2bf2(acc[0], acc[1]), f2bf2(acc[2], acc[3]));
  }
  TRACE_POINT(3);
  // The last out_proj workgroup clears the fold's counters for the next launch, counted in
  // two levels so that no counter line takes more than a few atomics: the last of each of
  // the L first-level lines counts on the top line.
  if (tid == 0) {
    const int L = min(kCoreCopies, a.O), line = ob % L, per = (a.O - line + L - 1) / L;
    if (add_agent(sy(a, kSyOutExit1 + line), 1u) == (uint32_t)(per - 1) &&
        add_agent(sy(a, kSyOutExit), 1u) == (uint32_t)(L - 1)) {
      for (int c = 0; c < kCoreCopies; ++c) {
        st_agent(sy(a, kSyCoreDone + c), 0u);
        st_agent(sy(a, kSyOutExit1 + c), 0u);
      }
      st_agent(sy(a, kSyOutExit), 0u);
    }
  }
}

// ---------------------------------------------------------------------------------------

// The launch arguments read through an address the compiler cannot see through (the kernel's
// argument segment, where Args is the only argument, passed through an empty asm): the
// fields a role reads are then loaded inside that role. Read through the parameter itself,
// the compiler may load them all at the kernel's entry, and the values the other roles need
// stay live in scalar registers across the whole role: in the multi-token launches that
// spilled scalar registers to a stack frame. The one-token launches, which have no spills,
// keep the parameter.
__device__ __forceinline__ const Args& role_args() {
  using KArgs = const __attribute__((address_space(4))) Args*;
  KArgs p = (KArgs)__builtin_amdgcn_kernarg_segment_ptr();
  asm volatile("" : "+s"(p));
  return *(const Args*)p;
}

// FOLD is a template flag, not only a launch argument, so that the out_proj role's register
// tile does not raise the register count (and lower the occupancy) of the launches without it.
template <bool PACKED, int FMT, int DK, typename ST, bool FOLD, bool MULTI, bool DST = false>
__global__ __launch_bounds__(kThreads) void decode_kernel(Args a) {
  // verify steps of more than one token at head dim 128 take the chunked recurrence and its
  // larger shared arrays
  constexpr bool kChunked = MULTI && DK == 128;
  __shared__ union {
    ProjShared proj;
    std::conditional_t<kChunked, VerShared, RecShared> rec;
  } sh;
  const int b = blockIdx.x;
  TRACE_POINT(0);
  const int nn = a.R * a.P, nr = a.Rs * a.nv;
  if (b < nn) {
    if (FMT == kFmtMx4 && a.normed)
      quant_role(a, b);
    else if (FMT == kFmtMx4)
      norm_role<true>(a, b, &sh.proj.red[0][0]);
    else
      norm_rstd_role(a, b, &sh.proj.red[0][0]);
  } else if (b < nn + a.G) {
    proj_role<PACKED, FMT>(a, b - nn, sh.proj);
  } else if (b < nn + a.G + nr) {
    if constexpr (kChunked)
      rec_verify<ST>(role_args(), b - nn - a.G, sh.rec);
    else if constexpr (MULTI)  // (inlined as before: not by itself once the asm is there)
      [[clang::always_inline]] rec_role<DK, ST, MULTI, DST>(role_args(), b - nn - a.G, sh.rec);
    else
      rec_role<DK, ST, MULTI, DST>(a, b - nn - a.G, sh.rec);
  } else if (FOLD) {
    oproj_role<PACKED>(a, b - nn - a.G - nr, sh.proj);
  }
}

// tiled copy of [in_proj_qkvz; in_proj_ba]: block (t, j) = 64 lanes x 16 bytes, lane l
// holding row 16 t + l % 16 at k = 32 j + 8 (l / 16); rows past the end are zero
__global__ __launch_bounds__(64) void pack_kernel(const uint16_t* __restrict__ wq, const uint16_t* __restrict__ wb,
                                                  uint16_t* __restrict__ out, int H, int Tq, int Nq, int Nb, int ns) {
  const int j = blockIdx.x, t = blockIdx.y, l = threadIdx.x;
  const bool isq = t < Tq;
  const int row = (isq ? t : t - Tq) * 16 + (l & 15);
  uint4 v = make_uint4(0u, 0u, 0u, 0u);
  if (row < (isq ? Nq : Nb))
    v = *reinterpret_cast<const uint4*>((isq ? wq : wb) + (size_t)row * H + 32 * j + 8 * (l >> 4));
  // block of (tile t, step j): grouped per K range of ns steps for the first Tq tiles when
  // ns > 0 (see wptr), one run per tile otherwise
  size_t b = (size_t)t * (H / 32) + j;
  if (isq && ns > 0) {
    const int s = j / ns, jj = j - s * ns;
    b = (((size_t)s * (Tq >> 2) + (t >> 2)) * ns + jj) * 4 + (t & 3);
  }
  *reinterpret_cast<uint4*>(out + (b * 64 + l) * 8) = v;
}

// tiled copy of MXFP4 in_proj_qkvz codes: block (t, j) = 64 lanes x 16 bytes, lane l holding
// the 32 codes of row 16 t + l % 16 at k = 128 j + 32 (l / 16)
// index of block b of tile t when each K range holds nb blocks, grouped as
// [K range][group of 4 tiles][block of the range][tile of the group] (Tq tiles in all)
__device__ __forceinline__ size_t grouped_block(int t, int b, int nb, int Tq) {
  const int s = b / nb, bb = b - s * nb;
  return (((size_t)s * (Tq >> 2) + (t >> 2)) * nb + bb) * 4 + (t & 3);
}
__global__ __launch_bounds__(64) void pack_mx_codes_kernel(const uint8_t* __restrict__ wq, uint8_t* __restrict__ out,
                                                           int H, int Tq, int kr) {
  const int j = blockIdx.x, t = blockIdx.y, l = threadIdx.x, row = t * 16 + (l & 15);
  const uint4 v = *reinterpret_cast<const uint4*>(wq + (size_t)row * (H >> 1) + 64 * j + 16 * (l >> 4));
  *reinterpret_cast<uint4*>(out + (grouped_block(t, j, kr >> 7, Tq) * 64 + l) * 16) = v;
}

// tiled copy of MXFP4 in_proj_qkvz scales: block (t, U) = 64 lanes x 4 bytes, lane l's byte
// st holding the scale of row 16 t + l % 16, K step 4 U + st, quarter l / 16
__global__ __launch_bounds__(64) void pack_mx_scales_kernel(const uint8_t* __restrict__ ws, uint32_t* __restrict__ out,
                                                            int H, int Tq, int kr) {
  const int U = blockIdx.x, t = blockIdx.y, l = threadIdx.x, row = t * 16 + (l & 15), kb = l >> 4;
  const uint8_t* src = ws + (size_t)row * (H >> 5) + 16 * U;
  uint32_t d = 0;
#pragma unroll
  for (int st = 0; st < 4; ++st) d |= (uint32_t)src[4 * st + kb] << (8 * st);
  out[grouped_block(t, U, kr >> 9, Tq) * 64 + l] = d;
}

// tiled copy of MXFP6 in_proj_qkvz codes: unit (t, U) = 1.5 KiB, the 16-byte heads of the 64
// lanes' code runs, then their 8-byte tails; lane l holding the 32 codes (24 bytes) of row
// 16 t + l % 16 at k = 128 U + 32 (l / 16). The scales take the MXFP4 scale tiles' layout.
__global__ __launch_bounds__(64) void pack_mx6_codes_kernel(const uint8_t* __restrict__ wq, uint8_t* __restrict__ out,
                                                            int H, int Tq, int kr) {
  const int U = blockIdx.x, t = blockIdx.y, l = threadIdx.x, row = t * 16 + (l & 15);
  const uint8_t* src = wq + ((size_t)row * (H >> 5) + 4 * U + (l >> 4)) * 24;
  const u32x2_t p0 = *reinterpret_cast<const u32x2_t*>(src), p1 = *reinterpret_cast<const u32x2_t*>(src + 8);
  const u32x2_t p2 = *reinterpret_cast<const u32x2_t*>(src + 16);
  uint8_t* dst = out + grouped_block(t, U, kr >> 7, Tq) * 1536;
  *reinterpret_cast<u32x4_t*>(dst + 16 * l) = u32x4_t{p0[0], p0[1], p1[0], p1[1]};
  *reinterpret_cast<u32x2_t*>(dst + 1024 + 8 * l) = p2;
}

// bf16 weights -> MXFP6 E2M3 blocks of 32 ("vLLM PR #60833", a reviewer's comment proposing
// MXFP6, step 2): one thread per block. The block maximum rounded to 3 mantissa bits
// carries into the next binade exactly when its top 4 mantissa bits are all set, which for
// a bf16 maximum is bits 6..3 of its 7; the scale exponent is that binade's minus 2, clamped
// to [-126, 127]. Each |x| / 2^e (exact) is rounded to the nearest E2M3 magnitude with ties
// to the even code: rint of |x| / 2^e at the step of its binade (1/8 below 2, 1/4 below 4,
// 1/2 above) counts grid points, and the code follows from the count (n for steps of 1/8,
// n + 8 for 1/4, n + 16 for 1/2, as E2M3 codes grow by one per grid point). A zero code
// carries no sign. Codes go out packed, code i at bits 6i..6i+5 of the block's 24 bytes.
__global__ __launch_bounds__(kThreads) void mx6_round_kernel(const uint16_t* __restrict__ w, uint8_t* __restrict__ codes,
                                                             uint8_t* __restrict__ scales, long long nblk) {
  const long long b = (long long)blockIdx.x * kThreads + threadIdx.x;
  if (b >= nblk) return;
  const u32x4_t* src = reinterpret_cast<const u32x4_t*>(w + b * 32);
  uint32_t v[16];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const u32x4_t t = src[q];
    v[4 * q] = t[0];
    v[4 * q + 1] = t[1];
    v[4 * q + 2] = t[2];
    v[4 * q + 3] = t[3];
  }
  uint32_t m = 0;  // the largest magnitude, as bf16 bits (finite values order like their bits)
#pragma unroll
  for (int q = 0; q < 16; ++q) m = max(m, max(v[q] & 0x7fffu, (v[q] >> 16) & 0x7fffu));
  const int E = (int)(m >> 7) + ((m & 0x78u) == 0x78u ? 1 : 0);  // biased binade of the rounded maximum
  const int e = min(127, max(-126, E - 127 - 2));
  const float inv = __uint_as_float((uint32_t)(127 - e) << 23);  // 2^-e (e <= 126 for bf16 inputs)
  uint64_t out[3] = {0, 0, 0};
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const uint32_t h = (i & 1) ? (v[i >> 1] >> 16) : (v[i >> 1] & 0xffffu);
    const float x = bf2f((uint16_t)(h & 0x7fffu)) * inv;
    uint32_t c = x < 2.0f ? (uint32_t)__builtin_rintf(x * 8.0f)
               : x < 4.0f ? (uint32_t)__builtin_rintf(x * 4.0f) + 8u
                          : (uint32_t)__builtin_rintf(x * 2.0f) + 16u;
    c = min(c, 31u);
    if ((h & 0x8000u) && c) c |= 32u;
    const int bit = 6 * i;
    out[bit >> 6] |= (uint64_t)c << (bit & 63);
    if ((bit & 63) > 58) out[(bit >> 6) + 1] |= (uint64_t)c >> (64 - (bit & 63));
  }
  uint64_t* dst = reinterpret_cast<uint64_t*>(codes + b * 24);
  dst[0] = out[0];
  dst[1] = out[1];
  dst[2] = out[2];
  scales[b] = (uint8_t)(e + 127);
}

// rows of bf16 -> MXFP4 codes [rows, cols/2] (low nibble = even element) and e8m0 scales
// [rows, cols/32], with the quantiser of the decode kernel; one workgroup per row
// A plain read stream, the reference the block's bandwidth is compared with (not a step of
// the block): every 16-byte word of src is read once, kStreamLoads per thread all in flight
// together. Workgroup b reads the 32 KiB from 32 KiB b on (thread t the words 2048 b + 256 u
// + t, u < kStreamLoads, so each wave's 64 loads at one u are one contiguous KiB; measured
// 3 % faster than interleaving the workgroups, and 4 or 8 loads per thread beat 16), and the
// words are folded by XOR into one word per workgroup, stored to sink[b] (the result keeps
// every load).
constexpr int kStreamLoads = 8;
__global__ __launch_bounds__(kThreads) void read_stream_kernel(const u32x4_t* __restrict__ src, long long n16,
                                                               uint32_t* __restrict__ sink) {
  const long long stride = kThreads, i0 = (long long)blockIdx.x * kThreads * kStreamLoads + threadIdx.x;
  u32x4_t v[kStreamLoads];
#pragma unroll
  for (int u = 0; u < kStreamLoads; ++u) {
    const long long i = i0 + u * stride;
    v[u] = i < n16 ? __builtin_nontemporal_load(src + i) : u32x4_t{0u, 0u, 0u, 0u};
  }
  uint32_t x = 0;
#pragma unroll
  for (int u = 0; u < kStreamLoads; ++u) x ^= (v[u][0] ^ v[u][1]) ^ (v[u][2] ^ v[u][3]);
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x ^= (uint32_t)__shfl_xor((int)x, m, 64);
  __shared__ uint32_t wx[kThreads / 64];
  if ((threadIdx.x & 63) == 0) wx[threadIdx.x >> 6] = x;
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x] = (wx[0] ^ wx[1]) ^ (wx[2] ^ wx[3]);
}

__global__ __launch_bounds__(kThreads) void mx_quant_kernel(const uint16_t* __restrict__ x, uint32_t* __restrict__ codes,
                                                            uint8_t* __restrict__ scales, int cols, int ceil) {
  const int row = blockIdx.x, nchunk = cols >> 3;
  for (int i = threadIdx.x; i < nchunk; i += kThreads) {
    // chunks of one 32-block sit on 4 consecutive lanes, which are active together
    const uint4 q = *reinterpret_cast<const uint4*>(x + (size_t)row * cols + 8 * i);
    const uint32_t v[4] = {q.x, q.y, q.z, q.w};
    uint32_t eb;
    codes[(size_t)row * nchunk + i] = mx_quant8(v, eb, ceil);
    if ((i & 3) == 0) scales[(size_t)row * (cols >> 5) + (i >> 2)] = (uint8_t)eb;
  }
}

}  // namespace

// The scratch of gdn_block_decode_noalloc: one fixed device array, which the code object
// loader places on every GPU the library runs on (held until the process ends). The
// hand-off counters take its first kStaticSyncBytes (the same offset for every handle, so
// handles of different shapes can use it one after another: each launch leaves every
// counter at zero); the activation image and the split partials follow. In host code the
// array's name is not a device address: the address is looked up once per device
// (static_scratch) and only that is passed to kernels and copies.
constexpr size_t kStaticScratchBytes = size_t(8) << 20;
constexpr size_t kStaticSyncBytes = size_t(64) << 10;
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

// =======================================================================================
// host side: the C ABI

namespace {
// the scratch pointers one launch uses: a handle's own allocation, or the static array
struct Scratch {
  uint16_t* xn;
  uint32_t* xq;
  uint32_t* xqs;
  float* part;
  uint32_t* sync;
};
}  // namespace

struct gdn_block {
  gdn_block_config cfg;
  int device;
  int nq, nb, cd, tq, tb, t, splits, steps, sync_words;
  int pw;             // floats per row of the split partials (whole 128-byte lines)
  int spin;           // poll limit of the bounded waits
  int cus;            // compute units of the device
  int kr;             // K range of a projection workgroup
  bool fold;          // out_proj folded in
  int o, ko;          // out_proj workgroups (4 tiles of 16 columns of H each) and K (nv * dv)
  int fmt;            // kFmtBf16, kFmtMx4 or kFmtMx6 (the in_proj_qkvz format)
  bool mx;            // MXFP4: the activations are quantised too (a second scratch image)
  void* scratch;       // the handle's own allocation: [data | sync words]
  size_t data_bytes;   // activation image and partials, at offsets o_* of a data base
  size_t o_xn, o_part, o_xq, o_xqs;
  Scratch own;
  uint32_t* sync;      // == own.sync
  std::string err;
};

namespace {

thread_local std::string g_create_error;

// per device: the address of the static scratch array (null until looked up), or why the
// lookup failed
constexpr int kMaxDevices = 64;
std::mutex g_static_mu;
void* g_static_ptr[kMaxDevices];
std::string g_static_why[kMaxDevices];

// Looks up (once per device, with that device current) the device address of the static
// scratch array, and clears its counter lines, which must start at zero.
void static_scratch_setup(int dev) {
  if (dev < 0 || dev >= kMaxDevices) return;
  std::lock_guard<std::mutex> lock(g_static_mu);
  if (g_static_ptr[dev] || !g_static_why[dev].empty()) return;
  void* ptr = nullptr;
  hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
  if (e == hipSuccess) e = hipMemset(ptr, 0, kStaticSyncBytes);
  if (e == hipSuccess) e = hipDeviceSynchronize();
  if (e == hipSuccess)
    g_static_ptr[dev] = ptr;
  else
    g_static_why[dev] = std::string("the static scratch of device ") + std::to_string(dev) +
                        " could not be set up: " + hipGetErrorString(e);
}

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// K range of a projection workgroup: the largest divisor of H up to kKr in whole units
// (4 waves x 32-wide bf16 steps, or 512 K for MXFP4 and MXFP6, whose scale dwords cover
// 512 K); 0 if there is none
int k_range(int H, bool mx) {
  const int unit = mx ? 512 : 128;
  for (int kr = kKr; kr >= unit; kr -= unit)
    if (H % kr == 0) return kr;
  return 0;
}

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
  const bool scaled = c->qkvz_format == GDN_FMT_MXFP4 || c->qkvz_format == GDN_FMT_MXFP6;
  if (c->qkvz_format != GDN_FMT_BF16 && !scaled)
    add("qkvz_format must be GDN_FMT_BF16, GDN_FMT_MXFP4 or GDN_FMT_MXFP6");
  if (scaled && c->hidden % 512 != 0)
    add(std::string(c->qkvz_format == GDN_FMT_MXFP4 ? "MXFP4" : "MXFP6") +
        " in_proj_qkvz needs hidden to be a multiple of 512 (got " + std::to_string(c->hidden) + ")");
  if (c->hidden > 0 && c->hidden % 256 == 0) {
    const int kr = k_range(c->hidden, scaled);
    if (kr == 0 || c->hidden / kr > kMaxSplits)
      add("hidden must split into at most " + std::to_string(kMaxSplits) + " K ranges of a multiple of " +
          (scaled ? "512" : "128") + " up to 1024 (got " + std::to_string(c->hidden) + ")");
  }
  if (c->ssm_state_dtype != GDN_STATE_F32 && c->ssm_state_dtype != GDN_STATE_BF16)
    add("ssm_state_dtype must be GDN_STATE_F32 or GDN_STATE_BF16");
  if (c->has_residual != 0 && c->has_residual != 1) add("has_residual must be 0 or 1");
  if (c->input_normed != 0 && c->input_normed != 1) add("input_normed must be 0 or 1");
  if (c->input_normed == 1 && c->has_residual == 1)
    add("input_normed takes the norm's output as x: has_residual must be 0");
  if (c->fold_out_proj != 0 && c->fold_out_proj != 1) add("fold_out_proj must be 0 or 1");
  if (c->mx_scale_rule != GDN_MXSCALE_ROUNDED_MAX && c->mx_scale_rule != GDN_MXSCALE_CEIL)
    add("mx_scale_rule must be GDN_MXSCALE_ROUNDED_MAX or GDN_MXSCALE_CEIL");
  if (c->fold_out_proj == 1) {
    const long long kv = (long long)c->num_v_heads * c->head_v_dim;
    if (kv % 128 != 0 || kv > 1024)
      add("fold_out_proj needs num_v_heads * head_v_dim to be a multiple of 128 up to 1024 (got " +
          std::to_string(kv) + ")");
  }
  auto bad_eps = [](float e) { return !(e > 0.0f) || !std::isfinite(e); };
  if (bad_eps(c->norm_eps) || bad_eps(c->gated_norm_eps) || bad_eps(c->l2norm_eps))
    add("every eps must be positive and finite");
  return why;
}

int fail(gdn_block* b, int code, const std::string& msg) {
  b->err = msg;
  return code;
}

template <bool PACKED, int FMT, int DK, typename ST>
void launch_st(const gdn_block* b, const Args& a, int grid, hipStream_t st) {
  if (b->fold)
    hipLaunchKernelGGL((decode_kernel<PACKED, FMT, DK, ST, true, false>), dim3(grid), dim3(kThreads), 0, st, a);
  else if (DK == 128 && a.dst && a.Tk == 1)  // one token: the decode recurrence with its destination
    hipLaunchKernelGGL((decode_kernel<PACKED, FMT, DK, ST, false, false, DK == 128>), dim3(grid), dim3(kThreads), 0,
                       st, a);
  else if (a.dst)
    hipLaunchKernelGGL((decode_kernel<PACKED, FMT, DK, ST, false, true>), dim3(grid), dim3(kThreads), 0, st, a);
  else
    hipLaunchKernelGGL((decode_kernel<PACKED, FMT, DK, ST, false, false>), dim3(grid), dim3(kThreads), 0, st, a);
}

template <bool PACKED, int FMT, int DK>
void launch_dk(const gdn_block* b, const Args& a, int grid, hipStream_t st) {
  if (b->cfg.ssm_state_dtype == GDN_STATE_F32)
    launch_st<PACKED, FMT, DK, float>(b, a, grid, st);
  else
    launch_st<PACKED, FMT, DK, uint16_t>(b, a, grid, st);
}

template <bool PACKED, int FMT>
void launch_fmt(const gdn_block* b, const Args& a, int grid, hipStream_t st) {
  switch (b->cfg.head_k_dim) {
    case 32: launch_dk<PACKED, FMT, 32>(b, a, grid, st); break;
    case 64: launch_dk<PACKED, FMT, 64>(b, a, grid, st); break;
    default: launch_dk<PACKED, FMT, 128>(b, a, grid, st); break;
  }
}

template <bool PACKED>
void launch(const gdn_block* b, const Args& a, int grid, hipStream_t st) {
  if (b->fmt == kFmtMx4)
    launch_fmt<PACKED, kFmtMx4>(b, a, grid, st);
  else if (b->fmt == kFmtMx6)
    launch_fmt<PACKED, kFmtMx6>(b, a, grid, st);
  else
    launch_fmt<PACKED, kFmtBf16>(b, a, grid, st);
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
  b->tb = (b->nb + 15) / 16;
  b->t = b->tq + b->tb;
  // a partial row: the in_proj_qkvz channels (key-head groups of a multiple of 64 channels,
  // so whole 128-byte lines), then the b|a channels padded to whole lines
  b->pw = b->nq + (int)align_up((size_t)b->nb, 32);
  b->spin = kSpinLimit;
  b->steps = H / 32;
  b->fmt = cfg->qkvz_format == GDN_FMT_MXFP4 ? kFmtMx4 : cfg->qkvz_format == GDN_FMT_MXFP6 ? kFmtMx6 : kFmtBf16;
  b->mx = b->fmt == kFmtMx4;
  b->fold = cfg->fold_out_proj == 1;
  b->o = H / 64;
  b->ko = nv * dv;
  // K ranges: a projection workgroup stages the activations of its range in LDS, so the
  // range is the largest divisor of H up to kKr in whole units (32-wide bf16 steps grouped
  // by 4 waves, or 512 K with MXFP4 or MXFP6). The split count depends on the shape only,
  // never on the row count.
  const int kr = k_range(H, b->fmt != kFmtBf16);
  b->kr = kr;
  const int S = H / kr;
  b->splits = S;
  b->sync_words = (kSyGroup0 + nk * kGroupCopies + cfg->max_rows * nk) * kLine;

  const int R = cfg->max_rows;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align_up(off + bytes, 256);
    return o;
  };
  b->o_xn = take((size_t)R * H * 2);
  b->o_part = take((size_t)S * R * b->pw * 4);
  b->o_xq = b->mx ? take((size_t)R * H / 2) : 0;
  b->o_xqs = b->mx ? take((size_t)R * H / 32) : 0;
  b->data_bytes = off;
  const size_t o_sync = take((size_t)b->sync_words * 4);

  hipError_t e = hipGetDevice(&b->device);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&b->cus, hipDeviceAttributeMultiprocessorCount, b->device);
  if (e == hipSuccess) e = hipMalloc(&b->scratch, off);
  if (e == hipSuccess) e = hipMemset(b->scratch, 0, off);
  if (e == hipSuccess) e = hipDeviceSynchronize();
  if (e != hipSuccess) {
    g_create_error = std::string("gdn_block_create: HIP error: ") + hipGetErrorString(e);
    if (b->scratch) (void)hipFree(b->scratch);
    delete b;
    return GDN_E_HIP;
  }
  char* base = static_cast<char*>(b->scratch);
  b->own.xn = reinterpret_cast<uint16_t*>(base + b->o_xn);
  b->own.part = reinterpret_cast<float*>(base + b->o_part);
  b->own.sync = reinterpret_cast<uint32_t*>(base + o_sync);
  b->own.xq = b->mx ? reinterpret_cast<uint32_t*>(base + b->o_xq) : nullptr;
  b->own.xqs = b->mx ? reinterpret_cast<uint32_t*>(base + b->o_xqs) : nullptr;
  b->sync = b->own.sync;
  // the set-up of gdn_block_decode_noalloc on this device (a failure is reported there)
  static_scratch_setup(b->device);
  g_create_error.clear();
  *out = b;
  return GDN_OK;
}

namespace {
// tiled copy: [in_proj_qkvz tiles | (MXFP4, MXFP6) their scale blocks | in_proj_ba tiles |
// (fold) out_proj tiles]
size_t packed_qkvz_bytes(const gdn_block* b) {
  const size_t H = b->cfg.hidden;
  return b->fmt == kFmtMx4 ? (size_t)b->nq * H / 2
       : b->fmt == kFmtMx6 ? (size_t)b->nq * H * 3 / 4 : (size_t)b->tq * 16 * H * 2;
}
size_t packed_scale_bytes(const gdn_block* b) {
  return b->fmt != kFmtBf16 ? (size_t)b->nq * b->cfg.hidden / 32 : 0;
}
size_t packed_ba_bytes(const gdn_block* b) { return (size_t)b->tb * 16 * b->cfg.hidden * 2; }
size_t packed_out_bytes(const gdn_block* b) { return b->fold ? (size_t)b->cfg.hidden * b->ko * 2 : 0; }
}  // namespace

extern "C" size_t gdn_block_packed_weight_bytes(gdn_block_t b) {
  if (!b) return 0;
  return packed_qkvz_bytes(b) + packed_scale_bytes(b) + packed_ba_bytes(b) + packed_out_bytes(b);
}

extern "C" int gdn_block_pack_weights(gdn_block_t b, const gdn_block_weights* w, void* packed, void* stream) {
  if (!b) return GDN_E_INVALID_ARG;
  if (!w || !w->w_qkvz || !w->w_ba || !packed)
    return fail(b, GDN_E_INVALID_ARG, "gdn_block_pack_weights: w, w->w_qkvz, w->w_ba and packed must not be NULL");
  if (b->fmt != kFmtBf16 && !w->w_qkvz_scales)
    return fail(b, GDN_E_INVALID_ARG, "gdn_block_pack_weights: w->w_qkvz_scales must not be NULL for MXFP4 and MXFP6");
  if (b->fold && (!w->w_out || !aligned16(w->w_out)))
    return fail(b, GDN_E_INVALID_ARG, "gdn_block_pack_weights: w->w_out must be a 16-byte aligned pointer (fold_out_proj)");
  if (!aligned16(w->w_qkvz) || !aligned16(w->w_ba) || !aligned16(packed) ||
      (b->fmt != kFmtBf16 && !aligned16(w->w_qkvz_scales)))
    return fail(b, GDN_E_INVALID_ARG, "gdn_block_pack_weights: pointers must be 16-byte aligned");
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int H = b->cfg.hidden;
  uint8_t* out = static_cast<uint8_t*>(packed);
  uint16_t* out_ba = reinterpret_cast<uint16_t*>(out + packed_qkvz_bytes(b) + packed_scale_bytes(b));
  if (b->fmt == kFmtBf16) {
    hipLaunchKernelGGL(pack_kernel, dim3(b->steps, b->t), dim3(64), 0, st, static_cast<const uint16_t*>(w->w_qkvz),
                       static_cast<const uint16_t*>(w->w_ba), reinterpret_cast<uint16_t*>(out), H, b->tq, b->nq, b->nb,
                       b->kr / 32);
  } else {
    const uint8_t* codes = static_cast<const uint8_t*>(w->w_qkvz);
    if (b->fmt == kFmtMx4)
      hipLaunchKernelGGL(pack_mx_codes_kernel, dim3(H / 128, b->tq), dim3(64), 0, st, codes, out, H, b->tq, b->kr);
    else
      hipLaunchKernelGGL(pack_mx6_codes_kernel, dim3(H / 128, b->tq), dim3(64), 0, st, codes, out, H, b->tq, b->kr);
    hipLaunchKernelGGL(pack_mx_scales_kernel, dim3(H / 512, b->tq), dim3(64), 0, st,
                       static_cast<const uint8_t*>(w->w_qkvz_scales),
                       reinterpret_cast<uint32_t*>(out + packed_qkvz_bytes(b)), H, b->tq, b->kr);
    // the b|a tiles in the bf16 tile layout (pack_kernel with no in_proj_qkvz tiles)
    hipLaunchKernelGGL(pack_kernel, dim3(b->steps, b->tb), dim3(64), 0, st, static_cast<const uint16_t*>(w->w_ba),
                       static_cast<const uint16_t*>(w->w_ba), out_ba, H, 0, 0, b->nb, 0);
  }
  if (b->fold)  // W_out [H, nv*dv] in the same 16-row tiles, after the b|a tiles
    hipLaunchKernelGGL(pack_kernel, dim3(b->ko / 32, 4 * b->o), dim3(64), 0, st, static_cast<const uint16_t*>(w->w_out),
                       static_cast<const uint16_t*>(w->w_out),
                       reinterpret_cast<uint16_t*>(out + packed_qkvz_bytes(b) + packed_scale_bytes(b) + packed_ba_bytes(b)),
                       b->ko, 4 * b->o, H, 0, 0);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(b, GDN_E_HIP, std::string("gdn_block_pack_weights: ") + hipGetErrorString(e));
  return GDN_OK;
}

namespace {
// one launch over `rows` sequences of `tokens` tokens each (decode: tokens = 1, dst_idx null)
int decode_impl(gdn_block* b, const Scratch& sc, const void* x, void* residual, const gdn_block_weights* w,
                void* conv_state, void* ssm_state, const int32_t* state_idx, const int32_t* dst_idx, int32_t rows,
                int32_t tokens, void* core_out, void* out, void* stream) {
  const gdn_block_config& c = b->cfg;
  if (tokens < 1 || tokens > c.max_rows)
    return fail(b, GDN_E_INVALID_ARG, "gdn_block_verify: tokens must be in 1.." + std::to_string(c.max_rows) +
                                          " (got " + std::to_string(tokens) + ")");
  if (rows < 0 || (long long)rows * tokens > c.max_rows)
    return fail(b, GDN_E_INVALID_ARG,
                std::string(tokens > 1 || dst_idx ? "gdn_block_verify: rows * tokens" : "gdn_block_decode: rows") +
                    " must be in 0.." + std::to_string(c.max_rows) + " (got " + std::to_string(rows) +
                    (tokens > 1 ? " x " + std::to_string(tokens) : std::string()) + ")");
  if (!w) return fail(b, GDN_E_INVALID_ARG, "gdn_block_decode: weights must not be NULL");
  if (b->fold) {
    if (!out || !aligned16(out))
      return fail(b, GDN_E_INVALID_ARG, "gdn_block_decode_with_out_proj: out must be a 16-byte aligned pointer");
    if (!w->w_proj_packed && (!w->w_out || !aligned16(w->w_out)))
      return fail(b, GDN_E_INVALID_ARG, "gdn_block_decode_with_out_proj: w_out must be a 16-byte aligned pointer");
  }
  const bool packed = w->w_proj_packed != nullptr;
  const bool normed = c.input_normed == 1;
  const bool scaled = b->fmt != kFmtBf16;
  const void* scales = (scaled && !packed) ? w->w_qkvz_scales : x;  // checked only when read
  const void* res_p = normed ? x : residual;                     // not read with a normed input
  const void* nw_p = normed ? x : w->norm_w;
  const void* ptrs[] = {x, res_p, conv_state, ssm_state, state_idx, core_out, nw_p,
                        packed ? w->w_proj_packed : w->w_qkvz, packed ? w->w_proj_packed : w->w_ba,
                        w->conv_w, w->A_log, w->dt_bias, w->gated_norm_w, scales};
  const char* names[] = {"x", normed ? "x" : "residual", "conv_state", "ssm_state", "state_idx", "core_out",
                         normed ? "x" : "norm_w",
                         packed ? "w_proj_packed" : "w_qkvz", packed ? "w_proj_packed" : "w_ba", "conv_w",
                         "A_log", "dt_bias", "gated_norm_w", (scaled && !packed) ? "w_qkvz_scales" : "x"};
  for (size_t i = 0; i < sizeof(ptrs) / sizeof(ptrs[0]); ++i) {
    if (!ptrs[i]) return fail(b, GDN_E_INVALID_ARG, std::string("gdn_block_decode: ") + names[i] + " is NULL");
    if (!aligned16(ptrs[i]))
      return fail(b, GDN_E_INVALID_ARG, std::string("gdn_block_decode: ") + names[i] + " is not 16-byte aligned");
  }
  if (dst_idx && !aligned16(dst_idx))
    return fail(b, GDN_E_INVALID_ARG, "gdn_block_verify: dst_idx is not 16-byte aligned");
  if (rows == 0) return GDN_OK;

  Args a;
  a.x = static_cast<const uint16_t*>(x);
  a.residual = static_cast<uint16_t*>(residual);
  a.norm_w = static_cast<const uint16_t*>(w->norm_w);
  a.wq = static_cast<const uint16_t*>(w->w_qkvz);
  a.wb = static_cast<const uint16_t*>(w->w_ba);
  a.wpk = static_cast<const uint16_t*>(w->w_proj_packed);
  a.wpk_sc = packed && scaled ? reinterpret_cast<const uint32_t*>(static_cast<const uint8_t*>(w->w_proj_packed) +
                                                                 packed_qkvz_bytes(b))
                             : nullptr;
  a.wpk_ba = packed ? reinterpret_cast<const uint16_t*>(static_cast<const uint8_t*>(w->w_proj_packed) +
                                                        packed_qkvz_bytes(b) + packed_scale_bytes(b))
                    : nullptr;
  a.wqc = scaled ? static_cast<const uint8_t*>(w->w_qkvz) : nullptr;
  a.wqs = scaled ? static_cast<const uint8_t*>(w->w_qkvz_scales) : nullptr;
  a.conv_w = static_cast<const uint16_t*>(w->conv_w);
  a.conv_state = static_cast<uint16_t*>(conv_state);
  a.ssm = ssm_state;
  a.idx = state_idx;
  a.dst = dst_idx;
  a.A_log = w->A_log;
  a.dt_bias = static_cast<const uint16_t*>(w->dt_bias);
  a.gnw = static_cast<const uint16_t*>(w->gated_norm_w);
  a.core = static_cast<uint16_t*>(core_out);
  a.fold = b->fold ? 1 : 0;
  a.O = b->fold ? b->o : 0;
  a.Ko = b->ko;
  a.out = static_cast<uint16_t*>(out);
  a.wo = static_cast<const uint16_t*>(w->w_out);
  a.wo_pk = packed ? reinterpret_cast<const uint16_t*>(static_cast<const uint8_t*>(w->w_proj_packed) +
                                                       packed_qkvz_bytes(b) + packed_scale_bytes(b) + packed_ba_bytes(b))
                   : nullptr;
  a.xn = sc.xn;
  a.xq = sc.xq;
  a.xqs = sc.xqs;
  a.part = sc.part;
  a.sync = sc.sync;
  a.H = c.hidden;
  a.R = rows * tokens;
  a.Rs = rows;
  a.Tk = tokens;
  a.has_res = c.has_residual;
  a.normed = normed ? 1 : 0;
  // norm workgroups per row: the MXFP4 image is made by ceil(H / 2048) of them, 2048 columns
  // each; otherwise one publishes the row's rstd
  // (a normed input has none, except MXFP4 past 2 rows: quantiser workgroups, 2048 columns each)
  const int p_mx = (c.hidden / 8 + kThreads - 1) / kThreads;
  a.P = normed ? (b->fmt == kFmtMx4 && rows * tokens > 2 ? p_mx : 0) : b->fmt == kFmtMx4 ? p_mx : 1;
  a.T = b->t;
  a.Tq = b->tq;
  a.Tb = b->tb;
  a.Nq = b->nq;
  a.Nb = b->nb;
  a.S = b->splits;
  a.Kr = b->kr;
  a.Gq = b->tq / 4 * b->splits;
  a.G = a.Gq + b->tb * b->splits;
  a.steps = b->steps;
  a.nk = c.num_k_heads;
  a.dk = c.head_k_dim;
  a.nv = c.num_v_heads;
  a.dv = c.head_v_dim;
  a.r = c.num_v_heads / c.num_k_heads;
  a.GW = 2 * c.head_k_dim + 2 * a.r * c.head_v_dim;
  a.Cd = b->cd;
  a.slots = c.num_state_slots;
  a.eps = c.norm_eps;
  a.l2eps = c.l2norm_eps;
  a.geps = c.gated_norm_eps;
  a.PW = b->pw;
  a.spin = b->spin;
  a.mx_ceil = c.mx_scale_rule == GDN_MXSCALE_CEIL ? 1 : 0;
  // The LDS fetch at launch pays when the projection workgroups all start at once (up to 2
  // per compute unit) and wait for the activations together; a larger grid streams in
  // several rounds with no such wait to hide (measured slower there).
  a.wlds = a.G <= 2 * b->cus ? 1 : 0;

  hipStream_t st = static_cast<hipStream_t>(stream);
  // no norm workgroups with a normed input; the out_proj workgroups last
  const int grid = a.R * a.P + a.G + rows * c.num_v_heads + a.O;
  if (packed)
    launch<true>(b, a, grid, st);
  else
    launch<false>(b, a, grid, st);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(b, GDN_E_HIP, std::string("gdn_block_decode: launch failed: ") + hipGetErrorString(e));
  return GDN_OK;
}
}  // namespace

extern "C" int gdn_block_decode(gdn_block_t b, const void* x, void* residual, const gdn_block_weights* w,
                                void* conv_state, void* ssm_state, const int32_t* state_idx, int32_t rows,
                                void* core_out, void* stream) {
  if (!b) return GDN_E_INVALID_ARG;
  if (b->fold)
    return fail(b, GDN_E_INVALID_ARG,
                "gdn_block_decode: this handle folds out_proj; call gdn_block_decode_with_out_proj");
  return decode_impl(b, b->own, x, residual, w, conv_state, ssm_state, state_idx, nullptr, rows, 1, core_out, nullptr,
                     stream);
}

extern "C" int gdn_block_decode_noalloc(gdn_block_t b, const void* x, void* residual, const gdn_block_weights* w,
                                        void* conv_state, void* ssm_state, const int32_t* state_idx, int32_t rows,
                                        void* core_out, void* stream) {
  if (!b) return GDN_E_INVALID_ARG;
  if (b->fold)
    return fail(b, GDN_E_INVALID_ARG,
                "gdn_block_decode_noalloc: this handle folds out_proj; call gdn_block_decode_with_out_proj");
  const int dev = b->device;
  void* base = nullptr;
  std::string why;
  if (dev >= 0 && dev < kMaxDevices) {
    std::lock_guard<std::mutex> lock(g_static_mu);
    base = g_static_ptr[dev];
    why = g_static_why[dev];
  }
  if (!base)
    return fail(b, GDN_E_HIP, "gdn_block_decode_noalloc: " +
                                  (why.empty() ? "no static scratch on device " + std::to_string(dev) : why));
  const size_t sync_bytes = (size_t)b->sync_words * 4;
  if (sync_bytes > kStaticSyncBytes || b->data_bytes > kStaticScratchBytes - kStaticSyncBytes)
    return fail(b, GDN_E_UNSUPPORTED,
                "gdn_block_decode_noalloc: this handle needs " + std::to_string(b->data_bytes) + " bytes of scratch and " +
                    std::to_string(sync_bytes) + " bytes of counters (max_rows " + std::to_string(b->cfg.max_rows) +
                    "); the static scratch holds " + std::to_string(kStaticScratchBytes - kStaticSyncBytes) + " and " +
                    std::to_string(kStaticSyncBytes) + ": create the handle with a smaller max_rows");
  char* data = static_cast<char*>(base) + kStaticSyncBytes;
  Scratch sc;
  sc.sync = static_cast<uint32_t*>(base);
  sc.xn = reinterpret_cast<uint16_t*>(data + b->o_xn);
  sc.part = reinterpret_cast<float*>(data + b->o_part);
  sc.xq = b->mx ? reinterpret_cast<uint32_t*>(data + b->o_xq) : nullptr;
  sc.xqs = b->mx ? reinterpret_cast<uint32_t*>(data + b->o_xqs) : nullptr;
  return decode_impl(b, sc, x, residual, w, conv_state, ssm_state, state_idx, nullptr, rows, 1, core_out, nullptr,
                     stream);
}

extern "C" int gdn_block_decode_with_out_proj(gdn_block_t b, const void* x, void* residual, const gdn_block_weights* w,
                                              void* conv_state, void* ssm_state, const int32_t* state_idx,
                                              int32_t rows, void* core_out, void* out, void* stream) {
  if (!b) return GDN_E_INVALID_ARG;
  if (!b->fold)
    return fail(b, GDN_E_INVALID_ARG,
                "gdn_block_decode_with_out_proj: this handle was created without fold_out_proj");
  return decode_impl(b, b->own, x, residual, w, conv_state, ssm_state, state_idx, nullptr, rows, 1, core_out, out,
                     stream);
}

extern "C" int gdn_block_verify(gdn_block_t b, const void* x, void* residual, const gdn_block_weights* w,
                                void* conv_state, void* ssm_state, const int32_t* src_idx, const int32_t* dst_idx,
                                int32_t rows, int32_t tokens, void* core_out, void* stream) {
  if (!b) return GDN_E_INVALID_ARG;
  if (!dst_idx) return fail(b, GDN_E_INVALID_ARG, "gdn_block_verify: dst_idx must not be NULL");
  if (b->fold)
    return fail(b, GDN_E_INVALID_ARG, "gdn_block_verify: not for a handle that folds out_proj");
  return decode_impl(b, b->own, x, residual, w, conv_state, ssm_state, src_idx, dst_idx, rows, tokens, core_out,
                     nullptr, stream);
}

extern "C" int gdn_block_check(gdn_block_t b, uint32_t* error_word) {
  if (!b || !error_word) return GDN_E_INVALID_ARG;
  void* st = nullptr;  // the static scratch of the handle's device, once set up
  if (b->device >= 0 && b->device < kMaxDevices) {
    std::lock_guard<std::mutex> lock(g_static_mu);
    st = g_static_ptr[b->device];
  }
  uint32_t v = 0, vs = 0;
  // every enqueued launch has ended, on every stream of the device
  hipError_t e = hipDeviceSynchronize();
  if (e == hipSuccess) e = hipMemcpy(&v, b->sync + (size_t)kSyError * kLine, 4, hipMemcpyDeviceToHost);
  if (e == hipSuccess && st)
    e = hipMemcpy(&vs, static_cast<uint32_t*>(st) + (size_t)kSyError * kLine, 4, hipMemcpyDeviceToHost);
  // A launch whose wait gave up may have left hand-off counters uncleared (their
  // clearing assumes that every workgroup arrived): clear all of them, and the word.
  if (e == hipSuccess && v) e = hipMemset(b->sync, 0, (size_t)b->sync_words * 4);
  if (e == hipSuccess && vs) e = hipMemset(st, 0, kStaticSyncBytes);
  if (e == hipSuccess && (v || vs)) e = hipDeviceSynchronize();
  if (e != hipSuccess) return fail(b, GDN_E_HIP, std::string("gdn_block_check: ") + hipGetErrorString(e));
  *error_word = v | vs;
  return GDN_OK;
}

extern "C" int gdn_block_set_spin_limit(gdn_block_t b, int32_t polls) {
  if (!b) return GDN_E_INVALID_ARG;
  if (polls < 0) return fail(b, GDN_E_INVALID_ARG, "gdn_block_set_spin_limit: polls must be >= 0");
  b->spin = polls;
  return GDN_OK;
}

#ifdef GDN_TRACE
// profiling builds only: copy the last launch's per-workgroup timestamps (kTraceSlots per block)
extern "C" int gdn_block_trace_copy(unsigned long long* host, size_t blocks) {
  if (blocks > (size_t)kTraceBlocks) blocks = kTraceBlocks;
  return hipMemcpyFromSymbol(host, HIP_SYMBOL(g_trace), blocks * kTraceSlots * sizeof(unsigned long long), 0,
                             hipMemcpyDeviceToHost) == hipSuccess ? GDN_OK : GDN_E_HIP;
}
#endif

extern "C" int gdn_mxfp4_quantize(const void* x, int32_t rows, int32_t cols, void* codes, void* scales,
                                  int32_t scale_rule, void* stream) {
  if (scale_rule != GDN_MXSCALE_ROUNDED_MAX && scale_rule != GDN_MXSCALE_CEIL) {
    g_create_error = "gdn_mxfp4_quantize: scale_rule must be GDN_MXSCALE_ROUNDED_MAX or GDN_MXSCALE_CEIL";
    return GDN_E_INVALID_ARG;
  }
  if (rows < 0 || cols <= 0 || cols % 32 != 0) {
    g_create_error = "gdn_mxfp4_quantize: rows must be >= 0 and cols a positive multiple of 32 (got rows " +
                     std::to_string(rows) + ", cols " + std::to_string(cols) + ")";
    return GDN_E_INVALID_ARG;
  }
  if (!x || !codes || !scales) {
    g_create_error = "gdn_mxfp4_quantize: x, codes and scales must not be NULL";
    return GDN_E_INVALID_ARG;
  }
  if (!aligned16(x) || (reinterpret_cast<uintptr_t>(codes) & 3u)) {
    g_create_error = "gdn_mxfp4_quantize: x must be 16-byte and codes 4-byte aligned";
    return GDN_E_INVALID_ARG;
  }
  if (rows == 0) return GDN_OK;
  hipLaunchKernelGGL(mx_quant_kernel, dim3(rows), dim3(kThreads), 0, static_cast<hipStream_t>(stream),
                     static_cast<const uint16_t*>(x), static_cast<uint32_t*>(codes), static_cast<uint8_t*>(scales),
                     (int)cols, scale_rule == GDN_MXSCALE_CEIL ? 1 : 0);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    g_create_error = std::string("gdn_mxfp4_quantize: launch failed: ") + hipGetErrorString(e);
    return GDN_E_HIP;
  }
  return GDN_OK;
}

extern "C" int gdn_mxfp6_round_weights(const void* w, int32_t rows, int32_t cols, void* codes, void* scales,
                                       void* stream) {
  if (rows < 0 || cols <= 0 || cols % 32 != 0) {
    g_create_error = "gdn_mxfp6_round_weights: rows must be >= 0 and cols a positive multiple of 32 (got rows " +
                     std::to_string(rows) + ", cols " + std::to_string(cols) + ")";
    return GDN_E_INVALID_ARG;
  }
  if (!w || !codes || !scales) {
    g_create_error = "gdn_mxfp6_round_weights: w, codes and scales must not be NULL";
    return GDN_E_INVALID_ARG;
  }
  if (!aligned16(w) || (reinterpret_cast<uintptr_t>(codes) & 7u)) {
    g_create_error = "gdn_mxfp6_round_weights: w must be 16-byte and codes 8-byte aligned";
    return GDN_E_INVALID_ARG;
  }
  if (rows == 0) return GDN_OK;
  const long long nblk = (long long)rows * (cols / 32);
  hipLaunchKernelGGL(mx6_round_kernel, dim3((unsigned)((nblk + kThreads - 1) / kThreads)), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), static_cast<const uint16_t*>(w), static_cast<uint8_t*>(codes),
                     static_cast<uint8_t*>(scales), nblk);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    g_create_error = std::string("gdn_mxfp6_round_weights: launch failed: ") + hipGetErrorString(e);
    return GDN_E_HIP;
  }
  return GDN_OK;
}

extern "C" int gdn_read_stream(const void* src, size_t bytes, uint32_t* sink, void* stream) {
  if (!src || !sink) {
    g_create_error = "gdn_read_stream: src and sink must not be NULL";
    return GDN_E_INVALID_ARG;
  }
  if (bytes == 0 || bytes % 16 != 0 || !aligned16(src) || (reinterpret_cast<uintptr_t>(sink) & 3u)) {
    g_create_error = "gdn_read_stream: bytes must be a positive multiple of 16, src 16-byte and sink 4-byte aligned "
                     "(got " + std::to_string(bytes) + " bytes)";
    return GDN_E_INVALID_ARG;
  }
  const long long n16 = (long long)(bytes / 16), per = (long long)kThreads * kStreamLoads;
  const long long grid = (n16 + per - 1) / per;  // = ceil(bytes / 32 KiB) workgroups and sink words
  if (grid > 0x7fffffffLL) {
    g_create_error = "gdn_read_stream: bytes too large";
    return GDN_E_INVALID_ARG;
  }
  hipLaunchKernelGGL(read_stream_kernel, dim3((unsigned)grid), dim3(kThreads), 0, static_cast<hipStream_t>(stream),
                     static_cast<const u32x4_t*>(src), n16, sink);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    g_create_error = std::string("gdn_read_stream: launch failed: ") + hipGetErrorString(e);
    return GDN_E_HIP;
  }
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
