// Device helpers shared by the frame kernel and the sampler kernel.
//
// Cross-block communication inside one kernel launch uses device-scope
// relaxed atomics for its writes: on gfx950 they compile to global
// loads/stores with the sc1 cache-policy bit, which are coherent across the
// eight XCDs without the L2 write-back/invalidate that device-scope fences
// cost.  Two forms of hand-over:
// - flag barriers: ordering between a block's data stores and its arrival
//   flag comes from s_waitcnt vmcnt(0) (stores are counted by vmcnt on
//   gfx9-family parts) plus a workgroup barrier; readers only touch the data
//   after observing every flag;
// - tagged values (st_tagged): each value carries its launch's tag in the
//   same 8-byte atomic store, so a reader checks the tag of every value it
//   loaded and reloads the stale ones with sc1 loads; no flag is needed and
//   no stale copy is ever used, wherever it came from.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace s2f {

typedef unsigned int u32;
typedef unsigned long long u64;

constexpr int NWAVE = 8;             // waves per block
constexpr int NTHREADS = NWAVE * 64; // threads per block
constexpr int MMAX = 2;              // activation rows one launch processes per phase
constexpr int TOPK_MAX = 64;         // sampler candidate limit (one per lane)
constexpr u32 SPIN_LIMIT = 1u << 22; // bounded waits: far longer than any phase

// A context's watchdog words (u32 offsets into one 256-word buffer, each
// pair on separate cache lines): a barrier wait that gave up during the
// current launch, the blocks that have left the current launch, and the
// sticky status the host reads back.
constexpr int W_ERR = 0, W_EXITS = 64, W_STATUS = 128, W_WORDS = 256;

// Test hook carried by every launch: with give_up set, every block's first
// barrier waits for an epoch no block publishes and gives up after one poll
// (and a wait on tagged values gives up at once), so the failure path runs
// while every block still exits normally.
struct Watch {
  u32 give_up;
};

__device__ __forceinline__ float ld_coh(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int ld_coh(const int* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ u32 ld_coh(const u32* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ long long ld_coh(const long long* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ u64 ld_coh64(const void* p) {
  return __hip_atomic_load(reinterpret_cast<const u64*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float lo_f32(u64 v) { return __uint_as_float((u32)v); }
__device__ __forceinline__ float hi_f32(u64 v) { return __uint_as_float((u32)(v >> 32)); }
__device__ __forceinline__ void st_coh(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_coh(int* p, int v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_coh(u32* p, u32 v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_coh(long long* p, long long v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void atomic_add_coh(long long* p, long long v) {
  __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Tagged values: a float in the low word of an 8-byte word whose high word
// names the launch that wrote it.  The 8-byte atomic store is single-copy
// atomic, so a reader that sees the tag it expects also sees that launch's
// value; a reader can therefore wait on the data itself instead of on a
// separate flag written after it.
__device__ __forceinline__ void st_tagged(u64* p, float v, u32 tag) {
  __hip_atomic_store(p, ((u64)tag << 32) | (u64)__float_as_uint(v), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ bool tag_is(u64 t, u32 tag) { return (u32)(t >> 32) == tag; }
__device__ __forceinline__ float tag_val(u64 t) { return __uint_as_float((u32)t); }
// First reads of tagged values use ordinary (L2-cacheable) loads, 16 bytes
// (two values) a lane where the layout allows: a copy that is not current
// (a line cached before its writer stored it) carries an older tag and is
// loaded again with coherent loads (ld_coh64), so a value is used only once
// its tag is current, wherever it came from.  The hardware never splits an
// aligned 8-byte word of such a load.
typedef unsigned long long u64x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void ld_tagged2(const u64* p, u64& a, u64& b) {
  const u64x2 v = *reinterpret_cast<const u64x2*>(p);
  a = v.x;
  b = v.y;
}
__device__ __forceinline__ u64 ld_tagged(const u64* p) { return *p; }

// s_waitcnt vmcnt(0) expcnt(7) lgkmcnt(15): this wave's vector memory
// operations (loads and stores) have completed.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float(((u32)b) << 16); }

// A pointer known to address global memory.  Weight pointers that reach a
// kernel through a table in device memory (rather than as kernel arguments)
// would otherwise be accessed with flat instructions, which also count
// against the LDS wait counter.
template <typename T>
__device__ __forceinline__ const __attribute__((address_space(1))) T* gbl(const T* p) {
  return (const __attribute__((address_space(1))) T*)p;
}

// 16 bytes of weights -> float values (8 bf16 or 4 f32)
template <typename WT> struct WTraits;
template <> struct WTraits<uint16_t> {
  static constexpr int EPL = 8;
  __device__ __forceinline__ static void unpack(const uint4& q, float* f) {
    f[0] = __uint_as_float(q.x << 16); f[1] = __uint_as_float(q.x & 0xFFFF0000u);
    f[2] = __uint_as_float(q.y << 16); f[3] = __uint_as_float(q.y & 0xFFFF0000u);
    f[4] = __uint_as_float(q.z << 16); f[5] = __uint_as_float(q.z & 0xFFFF0000u);
    f[6] = __uint_as_float(q.w << 16); f[7] = __uint_as_float(q.w & 0xFFFF0000u);
  }
  __device__ __forceinline__ static float one(const uint16_t* p, int i) { return bf16_to_f32(gbl(p)[i]); }
};
template <> struct WTraits<float> {
  static constexpr int EPL = 4;
  __device__ __forceinline__ static void unpack(const uint4& q, float* f) {
    f[0] = __uint_as_float(q.x); f[1] = __uint_as_float(q.y);
    f[2] = __uint_as_float(q.z); f[3] = __uint_as_float(q.w);
  }
  __device__ __forceinline__ static float one(const float* p, int i) { return gbl(p)[i]; }
};

// Weight-only int8 matrices: 16 signed weights per 16-byte load; each output
// row's float32 scale is applied to the row's dot product by the caller.
// The vectors of an int8 model (norm weights, embedding rows) are bf16
// (VecOf).
struct q8_t {
  int8_t v;
};
template <> struct WTraits<q8_t> {
  static constexpr int EPL = 16;
  __device__ __forceinline__ static void unpack(const uint4& q, float* f) {
    const u32 d[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) f[4 * i + j] = (float)(int)(signed char)(d[i] >> (8 * j));
  }
  __device__ __forceinline__ static float one(const q8_t* p, int i) { return (float)gbl(p)[i].v; }
};

// Element type of a model's vectors (norm weights, embedding rows).
template <typename WT> struct VecOf { using type = WT; };
template <> struct VecOf<q8_t> { using type = uint16_t; };

// Weights are read exactly once per decode step and never reused inside it:
// stream them with the non-temporal hint.
__device__ __forceinline__ uint4 ld_stream(const void* p) {
  const uint4* q = reinterpret_cast<const uint4*>(p);
  uint4 r;
  r.x = __builtin_nontemporal_load(&q->x);
  r.y = __builtin_nontemporal_load(&q->y);
  r.z = __builtin_nontemporal_load(&q->z);
  r.w = __builtin_nontemporal_load(&q->w);
  return r;
}

// Wave reductions.  Within each 16-lane row, DPP moves (quad permutations,
// then the half-row and row mirrors) combine values in registers; the four
// row results are then read out with readlane.  Every lane of the wave must
// be active.  Each combining step is commutative between the two lanes it
// pairs, so all lanes of a row hold bit-identical partial results and the
// returned value is the same in every lane.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, true));
}
constexpr int DPP_QUAD_1032 = 0xB1;      // quad_perm [1,0,3,2]
constexpr int DPP_QUAD_2301 = 0x4E;      // quad_perm [2,3,0,1]
constexpr int DPP_ROW_HALF_MIRROR = 0x141;
constexpr int DPP_ROW_MIRROR = 0x140;

// Value of lane (lane ^ J) for a constant J, without the LDS crossbar where
// the lane pattern allows: J = 1, 2 are quad permutations; J = 4, 8 stay
// inside a 16-lane row, so the lane takes the row shift by J in the direction
// of its partner (row_shl: lane + J, row_shr: lane - J); J = 16 is a swizzle
// (xor mask inside 32-lane halves); J = 32 goes through ds_bpermute.
template <int J>
__device__ __forceinline__ int xor_lane(int v, int lane) {
  if constexpr (J == 1) {
    return __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, true);
  } else if constexpr (J == 2) {
    return __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, true);
  } else if constexpr (J == 4 || J == 8) {
    const int up = __builtin_amdgcn_update_dpp(0, v, 0x100 + J, 0xF, 0xF, true);   // row_shl:J
    const int dn = __builtin_amdgcn_update_dpp(0, v, 0x110 + J, 0xF, 0xF, true);   // row_shr:J
    return (lane & J) ? dn : up;
  } else if constexpr (J == 16) {
    return __builtin_amdgcn_ds_swizzle(v, (0x10 << 10) | 0x1F);   // bitmask mode: xor 16, and 31
  } else {
    return __shfl_xor(v, J, 64);
  }
}
template <int J>
__device__ __forceinline__ float xor_lane_f(float v, int lane) {
  return __int_as_float(xor_lane<J>(__float_as_int(v), lane));
}

__device__ __forceinline__ float readlane_f(float v, int j) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), j));
}

__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_f<DPP_QUAD_1032>(v);
  v += dpp_f<DPP_QUAD_2301>(v);
  v += dpp_f<DPP_ROW_HALF_MIRROR>(v);
  v += dpp_f<DPP_ROW_MIRROR>(v);
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
  v = row16_sum(v);
  return (readlane_f(v, 0) + readlane_f(v, 16)) + (readlane_f(v, 32) + readlane_f(v, 48));
}
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp_f<DPP_QUAD_1032>(v));
  v = fmaxf(v, dpp_f<DPP_QUAD_2301>(v));
  v = fmaxf(v, dpp_f<DPP_ROW_HALF_MIRROR>(v));
  v = fmaxf(v, dpp_f<DPP_ROW_MIRROR>(v));
  return fmaxf(fmaxf(readlane_f(v, 0), readlane_f(v, 16)), fmaxf(readlane_f(v, 32), readlane_f(v, 48)));
}
__device__ __forceinline__ float wave_min(float v) {
  v = fminf(v, dpp_f<DPP_QUAD_1032>(v));
  v = fminf(v, dpp_f<DPP_QUAD_2301>(v));
  v = fminf(v, dpp_f<DPP_ROW_HALF_MIRROR>(v));
  v = fminf(v, dpp_f<DPP_ROW_MIRROR>(v));
  return fminf(fminf(readlane_f(v, 0), readlane_f(v, 16)), fminf(readlane_f(v, 32), readlane_f(v, 48)));
}

// SplitMix64 (Steele, Lea & Flood, OOPSLA 2014): add the golden gamma, then
// two xor-shift-multiply rounds and a final xor-shift, all modulo 2^64.
__device__ __forceinline__ u64 splitmix64(u64 x) {
  u64 z = x + 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

// Fixed-point accumulation of split-K partial sums: integer addition is
// associative, so the reduced value does not depend on the arrival order.
constexpr double FX_SCALE = 4294967296.0;          // 2^32
constexpr double FX_INV = 1.0 / 4294967296.0;
__device__ __forceinline__ long long to_fx(float v) { return __double2ll_rn((double)v * FX_SCALE); }
__device__ __forceinline__ float from_fx(long long a) { return (float)((double)a * FX_INV); }

}  // namespace s2f
