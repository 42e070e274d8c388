// Chunked single-pass scan of the gated linear recurrence
//     h_t = g_t * h_{t-1} + (1 - g_t) * x_t,   g_t = sigmoid(z_t),
// per channel, over the whole sequence (full-sequence recurrence with L = T:
// "RAT+: Train Dense, Infer Sparse", Fig. 1a; input-dependent gate and
// exponentially decaying memory: "Augmenting Attention with Exponentially
// Decaying Memory ...", section 2.1).  The pages' own prefill path uses an
// associative scan (RAT+ Fig. 2); this is a gfx950-native single-pass design.
//
// Decomposition.  Channels are contiguous in memory ([B][T][H][Dh]), so a lane
// owns NC adjacent channels and walks time sequentially; a wave covers 64*NC
// channels and kLW time steps; a block of kNW waves covers kNW*kLW steps (a
// "chunk") of one channel slab.  Every element is read once: z (fp32) and x
// (bf16 or fp32) go to registers, the local scan from a zero carry keeps
// (h_local, prod g) per step, and the true states follow as
//     h_t = h_local_t + (prod_{s<=t} g_s) * carry_in
// once the chunk's carry-in is known.
//
// Carry propagation across chunks is a decoupled look-back: blocks take
// chunk tickets from an atomic counter (slab fastest), publish their chunk
// aggregate (A = prod g, B = local end state) right after the local pass,
// then walk back over predecessors until one has published its inclusive end
// state.  Each published value is a 64-bit word {epoch:32, float bits:32}
// written with one relaxed agent-scope atomic store, so a reader validates
// every word by its tag alone: no fences, no per-call clearing.  A block
// waits only on lower tickets, which belong to blocks already running, so
// the waits always end; a bounded spin count still guards them and raises
// the workspace error flag instead of hanging.
#include "rat_internal.h"

namespace rat {
namespace {

constexpr int kLW = 16;              // time steps per wave
constexpr int kNW = 4;               // waves per block
constexpr int kChunkT = kLW * kNW;   // time steps per block
constexpr uint32_t kSpinLimit = 1u << 24;

// Raw vector of NC elements of type XT and its conversions.
template <typename XT, int NC> struct XVec;
template <> struct XVec<bf16_t, 4> {
  using raw = uint2;
  __device__ static raw load(const bf16_t* p) { return *reinterpret_cast<const uint2*>(p); }
  __device__ static float get(const raw& r, int c) {
    const uint32_t w = c < 2 ? r.x : r.y;
    return (c & 1) ? bf16_hi(w) : bf16_lo(w);
  }
  __device__ static void store(bf16_t* p, const float* v) {
    *reinterpret_cast<uint2*>(p) = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
  }
  __device__ static raw zero() { return make_uint2(0, 0); }
};
template <> struct XVec<bf16_t, 2> {
  using raw = uint32_t;
  __device__ static raw load(const bf16_t* p) { return *reinterpret_cast<const uint32_t*>(p); }
  __device__ static float get(const raw& r, int c) { return c ? bf16_hi(r) : bf16_lo(r); }
  __device__ static void store(bf16_t* p, const float* v) {
    *reinterpret_cast<uint32_t*>(p) = pack_bf16x2(v[0], v[1]);
  }
  __device__ static raw zero() { return 0u; }
};
template <> struct XVec<bf16_t, 1> {
  using raw = uint32_t;
  __device__ static raw load(const bf16_t* p) { return uint32_t(*p); }
  __device__ static float get(const raw& r, int) { return bf16_lo(r); }
  __device__ static void store(bf16_t* p, const float* v) {
    *p = bf16_t(pack_bf16x2(v[0], 0.f) & 0xffffu);
  }
  __device__ static raw zero() { return 0u; }
};
template <> struct XVec<float, 4> {
  using raw = float4;
  __device__ static raw load(const float* p) { return *reinterpret_cast<const float4*>(p); }
  __device__ static float get(const raw& r, int c) {
    return c == 0 ? r.x : c == 1 ? r.y : c == 2 ? r.z : r.w;
  }
  __device__ static void store(float* p, const float* v) {
    *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
  }
  __device__ static raw zero() { return make_float4(0.f, 0.f, 0.f, 0.f); }
};
template <> struct XVec<float, 2> {
  using raw = float2;
  __device__ static raw load(const float* p) { return *reinterpret_cast<const float2*>(p); }
  __device__ static float get(const raw& r, int c) { return c ? r.y : r.x; }
  __device__ static void store(float* p, const float* v) {
    *reinterpret_cast<float2*>(p) = make_float2(v[0], v[1]);
  }
  __device__ static raw zero() { return make_float2(0.f, 0.f); }
};
template <> struct XVec<float, 1> {
  using raw = float;
  __device__ static raw load(const float* p) { return *p; }
  __device__ static float get(const raw& r, int) { return r; }
  __device__ static void store(float* p, const float* v) { *p = v[0]; }
  __device__ static raw zero() { return 0.f; }
};

struct ScanArgs {
  ScanTensor ten[2];
  int B, T, H, Dh, C;
  int grid_mode;
  int n_slabs;        // ntensors * B * slabs_per_bt
  int slabs_per_bt;   // C / (64 * NC)
  uint64_t* agg_a;
  uint64_t* agg_b;
  uint64_t* incl;
  uint32_t* hdr;
  HeadTable heads;
};

__device__ __forceinline__ uint64_t tag_word(float v, uint32_t epoch) {
  return (uint64_t(epoch) << 32) | uint64_t(__float_as_uint(v));
}
__device__ __forceinline__ float word_value(uint64_t w) { return __uint_as_float(uint32_t(w)); }
__device__ __forceinline__ void publish(uint64_t* p, uint64_t w) {
  __hip_atomic_store(p, w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t peek(const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__global__ void scan_prologue(uint32_t* hdr) {
  if (threadIdx.x == 0) {
    uint32_t e = hdr[1] + 1u;
    if (e == 0u) e = 1u;
    hdr[0] = 0u;   // ticket counter
    hdr[1] = e;    // epoch of this call (hdr[2], the error word, is sticky)
  }
}

template <typename XT, int NC>
__global__ __launch_bounds__(kNW * 64) void scan_kernel(const ScanArgs a) {
  using V = XVec<XT, NC>;
  constexpr int SC = 64 * NC;   // channels per slab
  __shared__ uint32_t s_ticket;
  __shared__ float s_A[kNW][NC][64];
  __shared__ float s_B[kNW][NC][64];
  __shared__ float s_carry[kNW][NC][64];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  if (threadIdx.x == 0) s_ticket = atomicAdd(&a.hdr[0], 1u);
  __syncthreads();
  const uint32_t ticket = s_ticket;
  const uint32_t epoch = a.hdr[1];

  const int chunk = int(ticket / uint32_t(a.n_slabs));
  const int slab = int(ticket - uint32_t(chunk) * uint32_t(a.n_slabs));
  const int per_tensor = a.B * a.slabs_per_bt;
  const int ti = slab / per_tensor;
  const int rem = slab - ti * per_tensor;
  const int b = rem / a.slabs_per_bt;
  const int cs = rem - b * a.slabs_per_bt;
  const int ch = cs * SC + lane * NC;   // first channel of this lane in [0, C)
  const int h = ch / a.Dh;
  const int d = ch - h * a.Dh;
  const ScanTensor tn = ti == 0 ? a.ten[0] : a.ten[1];
  const int64_t C = a.C;
  const int T = a.T;
  const int t0 = chunk * kChunkT + wave * kLW;

  const XT* xp = static_cast<const XT*>(tn.x) + (int64_t)b * T * C + ch;
  const float* zp = tn.z + (int64_t)b * T * C + ch;

  // ---- load this wave's kLW steps (every element is read exactly once)
  typename V::raw xr[kLW];
  typename XVec<float, NC>::raw zr[kLW];
#pragma unroll
  for (int s = 0; s < kLW; ++s) {
    const int t = t0 + s;
    if (t < T) {
      xr[s] = V::load(xp + (int64_t)t * C);
      zr[s] = XVec<float, NC>::load(zp + (int64_t)t * C);
    } else {
      xr[s] = V::zero();
      zr[s] = XVec<float, NC>::zero();
    }
  }

  // ---- local scan from a zero carry
  float loc[kLW][NC], P[kLW][NC];
  float hl[NC], pp[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) { hl[c] = 0.f; pp[c] = 1.f; }
#pragma unroll
  for (int s = 0; s < kLW; ++s) {
    const bool live = (t0 + s) < T;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      float g, cc;
      gate_pair(XVec<float, NC>::get(zr[s], c), g, cc);
      if (!live) { g = 1.f; cc = 0.f; }   // identity step past the end
      hl[c] = g * hl[c] + cc * V::get(xr[s], c);
      pp[c] *= g;
      loc[s][c] = hl[c];
      P[s][c] = pp[c];
    }
  }
#pragma unroll
  for (int c = 0; c < NC; ++c) { s_A[wave][c][lane] = pp[c]; s_B[wave][c][lane] = hl[c]; }
  __syncthreads();

  // ---- wave 0: chunk aggregate, look-back, per-wave carries
  if (wave == 0) {
    float A[NC], Bv[NC], carry[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      A[c] = 1.f; Bv[c] = 0.f;
#pragma unroll
      for (int w = 0; w < kNW; ++w) {
        const float Aw = s_A[w][c][lane];
        Bv[c] = Aw * Bv[c] + s_B[w][c][lane];
        A[c] *= Aw;
      }
    }
    const int64_t widx = (int64_t)ticket * SC + lane * NC;
    if (chunk == 0) {
#pragma unroll
      for (int c = 0; c < NC; ++c)
        carry[c] = tn.h0 ? tn.h0[((int64_t)b * a.H + h) * a.Dh + d + c] : 0.f;
    } else {
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        publish(a.agg_a + widx + c, tag_word(A[c], epoch));
        publish(a.agg_b + widx + c, tag_word(Bv[c], epoch));
      }
      float accA[NC], accB[NC];
#pragma unroll
      for (int c = 0; c < NC; ++c) { accA[c] = 1.f; accB[c] = 0.f; }
      int j = chunk - 1;
      uint32_t spins = 0;
      bool done = false;
      while (!done) {
        const int64_t pidx = ((int64_t)j * a.n_slabs + slab) * SC + lane * NC;
        uint64_t wi[NC];
        bool ok = true;
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          wi[c] = peek(a.incl + pidx + c);
          ok = ok && uint32_t(wi[c] >> 32) == epoch;
        }
        if (ok) {
#pragma unroll
          for (int c = 0; c < NC; ++c) carry[c] = accA[c] * word_value(wi[c]) + accB[c];
          done = true;
        } else {
          uint64_t wa[NC], wb[NC];
          bool ok2 = true;
#pragma unroll
          for (int c = 0; c < NC; ++c) {
            wa[c] = peek(a.agg_a + pidx + c);
            wb[c] = peek(a.agg_b + pidx + c);
            ok2 = ok2 && uint32_t(wa[c] >> 32) == epoch && uint32_t(wb[c] >> 32) == epoch;
          }
          if (ok2) {
#pragma unroll
            for (int c = 0; c < NC; ++c) {
              accB[c] = accA[c] * word_value(wb[c]) + accB[c];
              accA[c] *= word_value(wa[c]);
            }
            --j;
          } else if (++spins > kSpinLimit) {
            atomicOr(&a.hdr[2], kErrScanSpin);
#pragma unroll
            for (int c = 0; c < NC; ++c) carry[c] = 0.f;
            done = true;
          } else {
            __builtin_amdgcn_s_sleep(1);
          }
        }
      }
    }
#pragma unroll
    for (int c = 0; c < NC; ++c) publish(a.incl + widx + c, tag_word(A[c] * carry[c] + Bv[c], epoch));
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      float cw = carry[c];
#pragma unroll
      for (int w = 0; w < kNW; ++w) {
        s_carry[w][c][lane] = cw;
        cw = s_A[w][c][lane] * cw + s_B[w][c][lane];
      }
    }
  }
  __syncthreads();

  // ---- finalize: true states, stores
  float cin[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) cin[c] = s_carry[wave][c][lane];

  const int D = a.grid_mode == kGridToken ? a.heads.dil[0] : a.heads.dil[h];
  // first grid position >= t0: smallest j >= t0 with (j + 1) % D == 0
  int next_grid = (t0 / D) * D + (D - 1);
  if (next_grid < t0) next_grid += D;
  XT* out_all = static_cast<XT*>(tn.out_all);
  XT* out_grid = static_cast<XT*>(tn.out_grid);
  const int64_t G_tok = D > 0 ? T / D : 0;

#pragma unroll
  for (int s = 0; s < kLW; ++s) {
    const int t = t0 + s;
    if (t < T) {
      float hv[NC];
#pragma unroll
      for (int c = 0; c < NC; ++c) hv[c] = loc[s][c] + P[s][c] * cin[c];
      if (out_all) V::store(out_all + ((int64_t)b * T + t) * C + ch, hv);
      if (out_grid && t == next_grid) {
        const int64_t i = (t + 1) / D - 1;
        int64_t off;
        if (a.grid_mode == kGridToken)
          off = (((int64_t)b * G_tok + i) * a.H + h) * a.Dh + d;
        else
          off = grid_row_offset(a.heads, a.B, b, h, i, a.Dh) + d;
        V::store(out_grid + off, hv);
        next_grid += D;
      }
      if (tn.h_last && t == T - 1) {
#pragma unroll
        for (int c = 0; c < NC; ++c) tn.h_last[((int64_t)b * a.H + h) * a.Dh + d + c] = hv[c];
      }
    }
  }
}

template <typename XT, int NC>
hipError_t launch_typed(const ScanArgs& a, int n_chunks, hipStream_t s) {
  const int blocks = n_chunks * a.n_slabs;
  hipLaunchKernelGGL((scan_kernel<XT, NC>), dim3(blocks), dim3(kNW * 64), 0, s, a);
  return hipGetLastError();
}

int pick_nc(int C) {
  if (C % 256 == 0) return 4;
  if (C % 128 == 0) return 2;
  return 1;
}

}  // namespace

size_t scan_workspace_bytes(int ntensors, int B, int T, int H, int Dh) {
  const int64_t C = (int64_t)H * Dh;
  const int64_t n_chunks = (T + kChunkT - 1) / kChunkT;
  const int64_t words = n_chunks * ntensors * (int64_t)B * C;   // one word per (chunk, channel)
  return sizeof(WsHeader) + 3 * (size_t)words * sizeof(uint64_t);
}

hipError_t launch_scan(const ScanPlan& p, hipStream_t s) {
  if (p.T <= 0 || p.B <= 0) return hipSuccess;
  ScanArgs a;
  a.ten[0] = p.ten[0];
  a.ten[1] = p.ntensors > 1 ? p.ten[1] : p.ten[0];
  a.B = p.B; a.T = p.T; a.H = p.H; a.Dh = p.Dh; a.C = p.H * p.Dh;
  a.grid_mode = p.grid_mode;
  a.heads = p.heads;
  const int nc = pick_nc(a.C);
  a.slabs_per_bt = a.C / (64 * nc);
  a.n_slabs = p.ntensors * p.B * a.slabs_per_bt;
  const int64_t n_chunks = (p.T + kChunkT - 1) / kChunkT;
  const int64_t words = n_chunks * p.ntensors * (int64_t)p.B * a.C;
  char* base = static_cast<char*>(p.ws);
  a.hdr = reinterpret_cast<uint32_t*>(base);
  a.agg_a = reinterpret_cast<uint64_t*>(base + sizeof(WsHeader));
  a.agg_b = a.agg_a + words;
  a.incl = a.agg_b + words;

  hipLaunchKernelGGL(scan_prologue, dim3(1), dim3(64), 0, s, a.hdr);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int nch = int(n_chunks);
  if (p.bf16) {
    if (nc == 4) return launch_typed<bf16_t, 4>(a, nch, s);
    if (nc == 2) return launch_typed<bf16_t, 2>(a, nch, s);
    return launch_typed<bf16_t, 1>(a, nch, s);
  }
  if (nc == 4) return launch_typed<float, 4>(a, nch, s);
  if (nc == 2) return launch_typed<float, 2>(a, nch, s);
  return launch_typed<float, 1>(a, nch, s);
}

}  // namespace rat
