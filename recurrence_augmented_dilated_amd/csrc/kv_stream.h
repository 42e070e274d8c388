// Streaming helpers shared by the decode-style kernels: one key row per
// group of Dh/8 lanes (eight elements per lane), dot products reduced with
// DPP inside the group, and a per-lane online softmax whose partial results
// merge exactly.
#pragma once

#include "rat_internal.h"

namespace rat {

// Eight consecutive elements of a row as fp32.
template <typename ET> struct Row8;
template <> struct Row8<bf16_t> {
  using raw = uint4;
  __device__ static raw load(const bf16_t* p) { return *reinterpret_cast<const uint4*>(p); }
  // a row read once per call (the cache streams): non-temporal, so that it
  // does not displace reused data from the caches
  __device__ static raw load_nt(const bf16_t* p) {
    typedef unsigned u4_t __attribute__((ext_vector_type(4)));
    const u4_t v = __builtin_nontemporal_load(reinterpret_cast<const u4_t*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
  }
  __device__ static raw zero() { return make_uint4(0, 0, 0, 0); }
  __device__ static void get(const raw& r, float* f) {
    f[0] = bf16_lo(r.x); f[1] = bf16_hi(r.x); f[2] = bf16_lo(r.y); f[3] = bf16_hi(r.y);
    f[4] = bf16_lo(r.z); f[5] = bf16_hi(r.z); f[6] = bf16_lo(r.w); f[7] = bf16_hi(r.w);
  }
  __device__ static void store(bf16_t* p, const float* f) {
    *reinterpret_cast<uint4*>(p) = make_uint4(pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]),
                                              pack_bf16x2(f[4], f[5]), pack_bf16x2(f[6], f[7]));
  }
  __device__ static float round(float x) { return round_bf16(x); }
  __device__ static void store1(bf16_t* p, float x) { *p = bf16_t(pack_bf16x2(x, 0.f) & 0xffffu); }
};
template <> struct Row8<float> {
  struct raw { float4 a, b; };
  __device__ static raw load(const float* p) {
    return raw{reinterpret_cast<const float4*>(p)[0], reinterpret_cast<const float4*>(p)[1]};
  }
  __device__ static raw load_nt(const float* p) {
    typedef float f4_t __attribute__((ext_vector_type(4)));
    const f4_t a = __builtin_nontemporal_load(reinterpret_cast<const f4_t*>(p));
    const f4_t b = __builtin_nontemporal_load(reinterpret_cast<const f4_t*>(p) + 1);
    return raw{make_float4(a.x, a.y, a.z, a.w), make_float4(b.x, b.y, b.z, b.w)};
  }
  __device__ static raw zero() { return raw{make_float4(0.f, 0.f, 0.f, 0.f), make_float4(0.f, 0.f, 0.f, 0.f)}; }
  __device__ static void get(const raw& r, float* f) {
    f[0] = r.a.x; f[1] = r.a.y; f[2] = r.a.z; f[3] = r.a.w;
    f[4] = r.b.x; f[5] = r.b.y; f[6] = r.b.z; f[7] = r.b.w;
  }
  __device__ static void store(float* p, const float* f) {
    reinterpret_cast<float4*>(p)[0] = make_float4(f[0], f[1], f[2], f[3]);
    reinterpret_cast<float4*>(p)[1] = make_float4(f[4], f[5], f[6], f[7]);
  }
  __device__ static float round(float x) { return x; }
  __device__ static void store1(float* p, float x) { *p = x; }
};

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xf, 0xf, true));
}

// Sum over groups of LPK adjacent lanes (LPK = 8 or 16); every lane gets the sum.
template <int LPK>
__device__ __forceinline__ float group_sum(float v) {
  if (LPK == 16) v += dpp<0x128>(v);   // row_ror:8
  v += dpp<0x141>(v);                  // row_half_mirror
  v += dpp<0x4E>(v);                   // quad_perm [2,3,0,1]
  v += dpp<0xB1>(v);                   // quad_perm [1,0,3,2]
  return v;
}

struct Soft {
  float m, l, acc[8];
};

__device__ __forceinline__ void soft_merge(Soft& x, float m2, float l2, const float* acc2) {
  const float mn = fmaxf(x.m, m2);
  if (mn == -INFINITY) return;
  const float f1 = __builtin_amdgcn_exp2f(x.m - mn);
  const float f2 = __builtin_amdgcn_exp2f(m2 - mn);
  x.l = x.l * f1 + l2 * f2;
#pragma unroll
  for (int i = 0; i < 8; ++i) x.acc[i] = x.acc[i] * f1 + acc2[i] * f2;
  x.m = mn;
}

// Online-softmax update with U keys (scores already in log2 units, -inf = none).
template <int U>
__device__ __forceinline__ void soft_update(Soft& x, const float* sc, const float (*vv)[8]) {
  float mx = sc[0];
#pragma unroll
  for (int u = 1; u < U; ++u) mx = fmaxf(mx, sc[u]);
  const float mn = fmaxf(x.m, mx);
  const float mu = mn == -INFINITY ? 0.f : mn;
  const float alpha = __builtin_amdgcn_exp2f(x.m - mu);
  float p[U];
  float ps = 0.f;
#pragma unroll
  for (int u = 0; u < U; ++u) { p[u] = __builtin_amdgcn_exp2f(sc[u] - mu); ps += p[u]; }
  x.l = x.l * alpha + ps;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    float a = x.acc[i] * alpha;
#pragma unroll
    for (int u = 0; u < U; ++u) a = fmaf(p[u], vv[u][i], a);
    x.acc[i] = a;
  }
  x.m = mn;
}

}  // namespace rat
