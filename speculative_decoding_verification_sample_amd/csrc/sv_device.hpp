// Device helpers for the gfx950 verify kernels: logit row geometry, 16-byte
// vector loads, bf16 widening, order-preserving keys, wave64 reductions and
// the split exponent used for tempered softmax masses.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sv_layout.hpp"

namespace sv {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// row / split geometry
// ---------------------------------------------------------------------------

// The elements [e0, e0 + n) of one split, cut into a scalar head (until the
// first 16-byte boundary), a body of 16-byte vectors and a scalar tail.
struct Span {
  const char *base;  // address of element e0
  int e0;            // first element (row-relative)
  int n;             // elements in the split
  int head;          // scalar elements before the body
  int nvec;          // 16-byte vectors in the body
  int tail;          // scalar elements after the body
};

__device__ __forceinline__ Span split_span(const char *row, int V, int s, int dtype) {
  const int es = elem_bytes(dtype);
  const int epv = 16 / es;
  Span sp;
  sp.e0 = s * split_elems(dtype);
  int e1 = min(V, sp.e0 + split_elems(dtype));
  sp.n = max(0, e1 - sp.e0);
  sp.base = row + (size_t)sp.e0 * es;
  uintptr_t a = reinterpret_cast<uintptr_t>(sp.base);
  int head = (int)(((16u - (unsigned)(a & 15u)) & 15u) / (unsigned)es);
  sp.head = min(head, sp.n);
  int rest = sp.n - sp.head;
  sp.nvec = rest / epv;
  sp.tail = rest - sp.nvec * epv;
  return sp;
}

// Scalar element handled by thread t (head first, then tail); -1 if none.
__device__ __forceinline__ int span_scalar_elem(const Span &sp, int t, int dtype) {
  if (t < sp.head) return t;
  int u = t - sp.head;
  if (u < sp.tail) return sp.head + sp.nvec * (16 / elem_bytes(dtype)) + u;
  return -1;
}

__device__ __forceinline__ const u32x4 *span_body(const Span &sp, int dtype) {
  return reinterpret_cast<const u32x4 *>(sp.base + (size_t)sp.head * elem_bytes(dtype));
}

// Generic split geometry: `per` elements per split (a multiple of 8).
__device__ __forceinline__ Span split_span_n(const char *row, int V, int s, int per, int dtype) {
  const int es = elem_bytes(dtype);
  const int epv = 16 / es;
  Span sp;
  sp.e0 = s * per;
  const int e1 = min(V, sp.e0 + per);
  sp.n = max(0, e1 - sp.e0);
  sp.base = row + (size_t)sp.e0 * es;
  const uintptr_t a = reinterpret_cast<uintptr_t>(sp.base);
  const int head = (int)(((16u - (unsigned)(a & 15u)) & 15u) / (unsigned)es);
  sp.head = min(head, sp.n);
  const int rest = sp.n - sp.head;
  sp.nvec = rest / epv;
  sp.tail = rest - sp.nvec * epv;
  return sp;
}

__device__ __forceinline__ u32x4 load_stream(const u32x4 *p) {
  return __builtin_nontemporal_load(p);
}

// ---------------------------------------------------------------------------
// element access
// ---------------------------------------------------------------------------

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Element i of a logit row, widened exactly to fp32.
__device__ __forceinline__ float load_elem(const char *row, size_t i, int dtype) {
  if (dtype == kBF16) {
    uint32_t h = reinterpret_cast<const uint16_t *>(row)[i];
    return __uint_as_float(h << 16);
  }
  return reinterpret_cast<const float *>(row)[i];
}

// Element k (0..epv-1) of a 16-byte vector.
__device__ __forceinline__ float vec_elem(const u32x4 &v, int k, int dtype) {
  if (dtype == kBF16) {
    uint32_t w = v[k >> 1];
    return (k & 1) ? bf16_hi(w) : bf16_lo(w);
  }
  return __uint_as_float(v[k]);
}

// ---------------------------------------------------------------------------
// order-preserving keys: larger value <-> larger key, -0.0 and +0.0 equal
// ---------------------------------------------------------------------------

__device__ __forceinline__ uint32_t key_of_f32(float f) {
  uint32_t u = __float_as_uint(f);
  uint32_t mag = u & 0x7FFFFFFFu;
  return (u >> 31) ? 0x80000000u - mag : 0x80000000u + mag;
}

__device__ __forceinline__ float f32_of_key(uint32_t k) {
  return k >= 0x80000000u ? __uint_as_float(k - 0x80000000u)
                          : __uint_as_float((0x80000000u - k) | 0x80000000u);
}

// ---------------------------------------------------------------------------
// tempered masses: exp((l - m) / T) = 2^((l - m) * k), k = log2(e) / T held as
// k_hi + k_lo so that the product carries ~1 ulp of error per element rather
// than the rounding of k itself (which would act like a shifted temperature).
// ---------------------------------------------------------------------------

__device__ __forceinline__ float exp2_fast(float a) { return __builtin_amdgcn_exp2f(a); }

// floor(x) as a signed integer in one instruction (v_cvt_flr_i32_f32, which
// the compiler does not form from floorf and a conversion): exact for |x| <
// 2^31, saturating beyond (-inf gives INT_MIN), NaN gives 0.
__device__ __forceinline__ int floor_to_int(float x) {
  int r;
  asm("v_cvt_flr_i32_f32 %0, %1" : "=v"(r) : "v"(x));
  return r;
}

// The upper 16 bits of x's fp32 pattern, raised by one unit where that is
// needed for the value they denote (low bits zero) not to lie below x:
// positive x with nonzero low bits.  NaN gives +inf.
__device__ __forceinline__ uint32_t f32_hi_up(float x) {
  const uint32_t b = __float_as_uint(x);
  if (x != x) return 0x7F80u;
  return (b >> 16) + ((b >> 31) == 0u && (b & 0xFFFFu) != 0u ? 1u : 0u);
}

__device__ __forceinline__ float tempered(float l, float m, Scale k) {
  float d = l - m;
  return exp2_fast(fmaf(d, k.hi, d * k.lo));
}

// ---------------------------------------------------------------------------
// wave64 reductions with DPP lane moves toward lane 63: pairs and quads
// (quad_perm), half rows and rows (mirrors), then the row broadcasts that
// carry row 0 into row 1, row 2 into row 3 and row 1 into rows 2 and 3; the
// total, read back from lane 63, lands in every lane.  Lanes that a move
// leaves out keep the identity.  Every lane must be active.
// ---------------------------------------------------------------------------

template <int CTRL, int ROWS = 0xF>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t old, uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)old, (int)v, CTRL, ROWS, 0xF, false);
}
template <int CTRL, int ROWS = 0xF>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t old, uint64_t v) {
  const uint32_t lo = dpp_u32<CTRL, ROWS>((uint32_t)old, (uint32_t)v);
  const uint32_t hi = dpp_u32<CTRL, ROWS>((uint32_t)(old >> 32), (uint32_t)(v >> 32));
  return ((uint64_t)hi << 32) | lo;
}
__device__ __forceinline__ uint64_t lane63_u64(uint64_t v) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, 63);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), 63);
  return ((uint64_t)hi << 32) | lo;
}
constexpr int kDppXor1 = 0xB1;       // quad_perm [1, 0, 3, 2]
constexpr int kDppXor2 = 0x4E;       // quad_perm [2, 3, 0, 1]
constexpr int kDppHalfMirror = 0x141;
constexpr int kDppMirror = 0x140;
constexpr int kDppBcast15 = 0x142;   // with rows 1 and 3 enabled
constexpr int kDppBcast31 = 0x143;   // with rows 2 and 3 enabled

__device__ __forceinline__ float wave_max(float v) {
  const uint32_t id = __float_as_uint(-INFINITY);
  v = fmaxf(v, __uint_as_float(dpp_u32<kDppXor1>(id, __float_as_uint(v))));
  v = fmaxf(v, __uint_as_float(dpp_u32<kDppXor2>(id, __float_as_uint(v))));
  v = fmaxf(v, __uint_as_float(dpp_u32<kDppHalfMirror>(id, __float_as_uint(v))));
  v = fmaxf(v, __uint_as_float(dpp_u32<kDppMirror>(id, __float_as_uint(v))));
  v = fmaxf(v, __uint_as_float(dpp_u32<kDppBcast15, 0xA>(id, __float_as_uint(v))));
  v = fmaxf(v, __uint_as_float(dpp_u32<kDppBcast31, 0xC>(id, __float_as_uint(v))));
  return __uint_as_float((uint32_t)__builtin_amdgcn_readlane((int)__float_as_uint(v), 63));
}

// fp64 sum in a fixed order (the same for every call)
__device__ __forceinline__ double wave_sum(double v) {
  auto bits = [](double x) { return (uint64_t)__double_as_longlong(x); };
  auto val = [](uint64_t x) { return __longlong_as_double((long long)x); };
  v += val(dpp_u64<kDppXor1>(0, bits(v)));
  v += val(dpp_u64<kDppXor2>(0, bits(v)));
  v += val(dpp_u64<kDppHalfMirror>(0, bits(v)));
  v += val(dpp_u64<kDppMirror>(0, bits(v)));
  v += val(dpp_u64<kDppBcast15, 0xA>(0, bits(v)));
  v += val(dpp_u64<kDppBcast31, 0xC>(0, bits(v)));
  return val(lane63_u64(bits(v)));
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
  auto mx = [](uint64_t a, uint64_t b) { return a > b ? a : b; };
  v = mx(v, dpp_u64<kDppXor1>(0, v));
  v = mx(v, dpp_u64<kDppXor2>(0, v));
  v = mx(v, dpp_u64<kDppHalfMirror>(0, v));
  v = mx(v, dpp_u64<kDppMirror>(0, v));
  v = mx(v, dpp_u64<kDppBcast15, 0xA>(0, v));
  v = mx(v, dpp_u64<kDppBcast31, 0xC>(0, v));
  return lane63_u64(v);
}

// Inclusive prefix sums over a wave (lanes in order): shifts by 1, 2, 4 and
// 8 inside each row of 16 lanes, then the row totals carried forward by the
// row broadcasts.  Every lane must be active.
__device__ __forceinline__ double wave_incl_scan(double v) {
  auto bits = [](double x) { return (uint64_t)__double_as_longlong(x); };
  auto val = [](uint64_t x) { return __longlong_as_double((long long)x); };
  v += val(dpp_u64<0x111>(0, bits(v)));  // row_shr:1
  v += val(dpp_u64<0x112>(0, bits(v)));  // row_shr:2
  v += val(dpp_u64<0x114>(0, bits(v)));  // row_shr:4
  v += val(dpp_u64<0x118>(0, bits(v)));  // row_shr:8
  v += val(dpp_u64<kDppBcast15, 0xA>(0, bits(v)));
  v += val(dpp_u64<kDppBcast31, 0xC>(0, bits(v)));
  return v;
}
__device__ __forceinline__ int wave_incl_scan(int v) {
  v += (int)dpp_u32<0x111>(0, (uint32_t)v);
  v += (int)dpp_u32<0x112>(0, (uint32_t)v);
  v += (int)dpp_u32<0x114>(0, (uint32_t)v);
  v += (int)dpp_u32<0x118>(0, (uint32_t)v);
  v += (int)dpp_u32<kDppBcast15, 0xA>(0, (uint32_t)v);
  v += (int)dpp_u32<kDppBcast31, 0xC>(0, (uint32_t)v);
  return v;
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

// ---------------------------------------------------------------------------
// cross-workgroup hand-off without whole-cache fences.  The 8 XCDs have their
// own L2s; an agent-scope fence writes back and invalidates a whole L2.
// Instead the few words that one workgroup hands to another are stored and
// loaded as agent-scope relaxed atomics (coherent across XCDs), and the
// producer waits for its stores to complete before it bumps the counter.
// ---------------------------------------------------------------------------

template <class T>
__device__ __forceinline__ void store_agent(T *p, T v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <class T>
__device__ __forceinline__ T load_agent(const T *p) {
  return __hip_atomic_load(const_cast<T *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Wait until every memory operation this lane issued has completed.
__device__ __forceinline__ void wait_memory() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Epoch tags.  Every call carries a fresh 64-bit epoch.  A producer stores
// its partial, waits for those stores to complete, then stores the epoch in
// the partial's tag word; a consumer polls the tags of the cells it needs
// and reads a cell only once its tag equals the current epoch.  Tags left by
// earlier calls (or whatever the workspace held) never match, so nothing has
// to clear the workspace, and no atomic read-modify-write is involved.
__device__ __forceinline__ void publish_tag(u64 *tag, u64 epoch) {
  wait_memory();  // the partial's stores are complete before the tag lands
  store_agent(tag, epoch);
}

// Bounded wait (about a second at most) until *tag == epoch; false on
// time-out.  Only ever used on work that has already been dispatched.
constexpr int kSpinLimit = 1 << 20;
__device__ __forceinline__ bool tag_wait(const u64 *tag, u64 epoch) {
  for (int it = 0; it < kSpinLimit; ++it) {
    if (load_agent(tag) == epoch) return true;
    __builtin_amdgcn_s_sleep(2);
  }
  return false;
}

// The whole workgroup waits for tags[0..n); false if any wait timed out.
__device__ __forceinline__ bool block_wait_tags(const u64 *tags, int n, u64 epoch, int *flag) {
  if (threadIdx.x == 0) *flag = 1;
  __syncthreads();
  bool ok = true;
  for (int i = threadIdx.x; i < n; i += blockDim.x) ok = ok && tag_wait(&tags[i], epoch);
  if (!ok) *flag = 0;
  __syncthreads();
  return *flag != 0;
}

// Self-validating 64-bit words: the epoch's low 32 bits ride in the low half
// of each word and a 32-bit payload in the high half, so one store publishes
// a value and one load both reads and validates it (no store-completion wait,
// no separate tag round trip). Relaxed stores to two addresses may become
// visible in either order, so a reader can meet one fresh word beside a stale
// one: every word therefore carries the full 32-bit tag on its own (a word
// left by an earlier call validates only if its call's epoch agrees in all 32
// low bits). An fp64 value travels as two such words (see split_f64).
// a 32-bit payload in the high word, the epoch's low 32 bits in the low word
__device__ __forceinline__ u64 pack_u32(uint32_t v, u64 epoch) {
  return ((u64)v << 32) | (epoch & 0xFFFFFFFFull);
}
__device__ __forceinline__ bool unpack_u32(u64 w, u64 epoch, uint32_t *v) {
  *v = (uint32_t)(w >> 32);
  return (w & 0xFFFFFFFFull) == (epoch & 0xFFFFFFFFull);
}
__device__ __forceinline__ float payload_f32(u64 w) { return __uint_as_float((uint32_t)(w >> 32)); }
// an fp64 value as an unevaluated sum hi + lo of two fp32 values (about 48
// significant bits; exact for the values here, which lie well inside fp32's range)
__device__ __forceinline__ void split_f64(double v, float *hi, float *lo) {
  *hi = (float)v;
  *lo = (float)(v - (double)*hi);
}
// two 16-bit indices (each -1 .. 65534) and the epoch's low 32 bits
__device__ __forceinline__ u64 pack_idx2(int a, int b, u64 epoch) {
  return ((epoch & 0xFFFFFFFFull) << 32) | ((u64)(unsigned)(a + 1) << 16) | (u64)(unsigned)(b + 1);
}
__device__ __forceinline__ bool unpack_idx2(u64 w, u64 epoch, int *a, int *b) {
  *a = (int)((w >> 16) & 0xFFFFull) - 1;
  *b = (int)(w & 0xFFFFull) - 1;
  return (w >> 32) == (epoch & 0xFFFFFFFFull);
}

__device__ __forceinline__ void spin_pause() { __builtin_amdgcn_s_sleep(2); }

}  // namespace sv
