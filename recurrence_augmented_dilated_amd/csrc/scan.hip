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
// "chunk") of one channel slab.  Every input element is read from HBM once
// and kept in registers as loaded (bf16/fp32 x, fp32 z): a first pass turns
// every z into c = 1 - g in place and folds the wave's steps into an
// aggregate (A = prod g, B = state reached from a zero carry), and once the
// chunk's carry-in is known a second pass re-runs the recurrence from it over
// the same registers (h - c h + c x: two FMAs per element, no second sigmoid
// and no rounded 1 - c) and stores the states.
//
// Carry propagation across chunks is a decoupled look-back.  Block b of the
// grid handles chunk b / n_slabs of slab b % n_slabs, publishes its chunk
// aggregate right after the first pass, then looks back over predecessors
// (same slab, earlier chunks) until one has published its inclusive end
// state.  Every thread owns one channel of the slab and reads a window of
// kWin predecessors per round trip.  Each published value is a 64-bit word
// {epoch:32, float bits:32} written with one relaxed agent-scope atomic
// store, so a reader validates every word by its tag alone: no fences, no
// per-call clearing.  Work is ordered by block index rather than by an
// atomic ticket (same-address device atomics serialise, about one per
// 60-70 ns on this part, which capped the scan at a few thousand blocks per
// 0.3 ms).  Waits cannot deadlock even if blocks were dispatched out of
// order: a thread that sees no progress from a predecessor for kFallbackSpins
// polls computes that predecessor's aggregate itself from its inputs and
// keeps walking back; chunk 0 needs nobody, so every wait ends.
#include "rat_internal.h"

namespace rat {
namespace {

constexpr int kLW = 16;              // time steps per wave
constexpr int kNW = 8;               // waves per block
constexpr int kChunkT = kLW * kNW;   // time steps per block
constexpr int kSegNW = 16;           // waves per segmented-scan block (one block per CU: no
                                     // wave-age skew between two resident blocks)
constexpr int kSegChunkT = kLW * kSegNW;   // time steps per segmented-scan chunk
static_assert(kSegChunkT % kChunkT == 0, "a segment chunk is whole plain chunks");
static_assert(kSegMinD >= kLW, "a grid-only wave holds at most one grid position");
constexpr int kWin = 2;              // predecessors read per look-back round trip
constexpr int kSparseMaxD = 32;      // largest D whose column grid is staged through LDS
constexpr uint32_t kFallbackSpins = 256;   // default polls before computing a predecessor locally
                                           // (the workspace header's poll_limit word overrides it)

// Hide a register value from the optimiser (an empty asm that "modifies"
// it), so that pass 2 recomputes the gates instead of keeping pass 1's.
__device__ __forceinline__ void opaque(uint32_t& v) { asm volatile("" : "+v"(v)); }
__device__ __forceinline__ void opaque(float& v) { asm volatile("" : "+v"(v)); }

// Raw vector of NC elements of type XT and its conversions.
template <typename XT, int NC> struct XVec;
template <> struct XVec<bf16_t, 2> {
  using raw = uint32_t;
  __device__ static raw load(const bf16_t* p) { return *reinterpret_cast<const uint32_t*>(p); }
  __device__ static raw load_nt(const bf16_t* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p));
  }
  __device__ static float get(const raw& r, int c) { return c ? bf16_hi(r) : bf16_lo(r); }
  __device__ static void store(bf16_t* p, const float* v) {
    *reinterpret_cast<uint32_t*>(p) = pack_bf16x2(v[0], v[1]);
  }
  __device__ static raw zero() { return 0u; }
  __device__ static void hide(raw& r) { opaque(r); }
};
template <> struct XVec<bf16_t, 1> {
  using raw = uint32_t;
  __device__ static raw load(const bf16_t* p) { return uint32_t(*p); }
  __device__ static raw load_nt(const bf16_t* p) { return uint32_t(__builtin_nontemporal_load(p)); }
  __device__ static float get(const raw& r, int) { return bf16_lo(r); }
  __device__ static void store(bf16_t* p, const float* v) {
    *p = bf16_t(pack_bf16x2(v[0], 0.f) & 0xffffu);
  }
  __device__ static raw zero() { return 0u; }
  __device__ static void hide(raw& r) { opaque(r); }
};
template <> struct XVec<float, 2> {
  using raw = float2;
  __device__ static raw load(const float* p) { return *reinterpret_cast<const float2*>(p); }
  __device__ static raw load_nt(const float* p) {
    typedef float f2_t __attribute__((ext_vector_type(2)));
    const f2_t v = __builtin_nontemporal_load(reinterpret_cast<const f2_t*>(p));
    return make_float2(v.x, v.y);
  }
  __device__ static float get(const raw& r, int c) { return c ? r.y : r.x; }
  __device__ static void store(float* p, const float* v) {
    *reinterpret_cast<float2*>(p) = make_float2(v[0], v[1]);
  }
  __device__ static raw zero() { return make_float2(0.f, 0.f); }
  __device__ static void hide(raw& r) { opaque(r.x); opaque(r.y); }
  __device__ static void set(raw& r, int c, float v) { (c ? r.y : r.x) = v; }
};
template <> struct XVec<float, 1> {
  using raw = float;
  __device__ static raw load(const float* p) { return *p; }
  __device__ static raw load_nt(const float* p) { return __builtin_nontemporal_load(p); }
  __device__ static float get(const raw& r, int) { return r; }
  __device__ static void store(float* p, const float* v) { *p = v[0]; }
  __device__ static raw zero() { return 0.f; }
  __device__ static void hide(raw& r) { opaque(r); }
  __device__ static void set(raw& r, int, float v) { r = v; }
};

// a + b for non-negative b, saturating at INT_MAX (row indices past the
// sequence only need to stay out of reach)
__device__ __forceinline__ int sat_add(int a, int b) {
  return a > 0x7fffffff - b ? 0x7fffffff : a + b;
}

// Stores into the transposed (column) layouts: four consecutive keys of one
// row, or one key.
__device__ __forceinline__ void store4(bf16_t* p, const float* v) {
  *reinterpret_cast<uint2*>(p) = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
}
__device__ __forceinline__ void store4(float* p, const float* v) {
  *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ void store1(bf16_t* p, float v) { *p = bf16_t(pack_bf16x2(v, 0.f) & 0xffffu); }
__device__ __forceinline__ void store1(float* p, float v) { *p = v; }

struct ScanArgs {
  ScanTensor ten[2];
  int B, T, H, Dh, C;
  int64_t tpad;       // row length of kAllHeadCol outputs
  int64_t p0;         // absolute position of input row 0
  int64_t all_row0;   // all-state row of input row 0
  int64_t arows;      // rows of kAllToken outputs
  int reset_every;    // > 0: the state restarts from zero at positions j with j % reset_every == 0
  int n_slabs;        // ntensors * B * slabs_per_bt
  int slabs_per_bt;   // C / (64 * NC)
  uint64_t* agg_a;
  uint64_t* agg_b;
  uint64_t* incl;
  uint32_t* hdr;
  float* part[2];     // segmented scan: (A, B) pairs per grid element and tensor
  int n_seg;          // segmented scan: segments per slab
  int seg_chunks;     // segmented scan: chunks per segment
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
    hdr[1] = e;    // epoch of this call (hdr[2], the error word, is sticky)
  }
}

// Aggregate (prod g, state from a zero carry) of chunk j for one channel,
// computed straight from the inputs: the look-back's fallback.
template <typename XT, bool RESET>
__device__ void chunk_aggregate(const XT* x, const float* z, int64_t C, int T, int j, int64_t p0, int reset,
                                float& A, float& Bv) {
  A = 1.f;
  Bv = 0.f;
  const int t_end = min(T, (j + 1) * kChunkT);
  for (int t = j * kChunkT; t < t_end; ++t) {
    const float c = gate_comp(z[(int64_t)t * C]);
    const bool restart = RESET && (p0 + t) % reset == 0;   // the carried state is dropped
    const float xv = sizeof(XT) == 2 ? bf16_to_f32(reinterpret_cast<const bf16_t*>(x)[(int64_t)t * C])
                                     : reinterpret_cast<const float*>(x)[(int64_t)t * C];
    Bv = restart ? c * xv : fmaf(c, xv, fmaf(-c, Bv, Bv));   // (1 - c) B + c x
    A = restart ? 0.f : fmaf(-A, c, A);
  }
}

// Carry into chunk `chunk` of a slab for channel cl of the slab (one thread
// per channel): publishes the chunk's aggregate (A, Bv), then walks back over
// the predecessors' published words until an inclusive state is found,
// folding in the aggregates on the way (or computing a silent predecessor's
// aggregate from its inputs after fallback_spins polls).  Chunk 0 starts
// from h0.
template <typename XT, bool RESET, int SC>
__device__ __forceinline__ float chunk_carry(const ScanArgs& a, const ScanTensor& tn, uint32_t ticket, int chunk,
                                             int slab, int b, int cs, int cl, float A, float Bv, uint32_t epoch,
                                             uint32_t fallback_spins) {
  const int64_t C = a.C;
  const int T = a.T;
  const int64_t widx = (int64_t)ticket * SC + cl;
  float carry = 0.f;
  if (chunk == 0) {
    const int chg = cs * SC + cl;
    const int hh = chg / a.Dh;
    carry = tn.h0 ? tn.h0[((int64_t)b * a.H + hh) * a.Dh + (chg - hh * a.Dh)] : 0.f;
  } else {
    publish(a.agg_a + widx, tag_word(A, epoch));
    publish(a.agg_b + widx, tag_word(Bv, epoch));
    float accA = 1.f, accB = 0.f;
    int j = chunk - 1;
    uint32_t spins = 0;
    bool done = false;
    while (!done) {
      uint64_t wi[kWin], wa[kWin], wb[kWin];
#pragma unroll
      for (int i = 0; i < kWin; ++i) {
        const int jj = j - i;
        if (jj >= 0) {
          const int64_t pidx = ((int64_t)jj * a.n_slabs + slab) * SC + cl;
          wi[i] = peek(a.incl + pidx);
          wa[i] = peek(a.agg_a + pidx);
          wb[i] = peek(a.agg_b + pidx);
        } else {
          wi[i] = wa[i] = wb[i] = 0;
        }
      }
      int used = 0;
      bool stop = false;
#pragma unroll
      for (int i = 0; i < kWin; ++i) {
        if (!stop && !done) {
          if (uint32_t(wi[i] >> 32) == epoch) {
            carry = accA * word_value(wi[i]) + accB;
            done = true;
          } else if (uint32_t(wa[i] >> 32) == epoch && uint32_t(wb[i] >> 32) == epoch) {
            accB = accA * word_value(wb[i]) + accB;
            accA *= word_value(wa[i]);
            ++used;
          } else {
            stop = true;
          }
        }
      }
      if (done) break;
      j -= used;
      if (used > 0) {
        spins = 0;
      } else if (++spins > fallback_spins) {
        // predecessor j shows no progress: fold its chunk in directly
        const int chg = cs * SC + cl;
        float Aj, Bj;
        chunk_aggregate<XT, RESET>(static_cast<const XT*>(tn.x) + (int64_t)b * T * C + chg,
                                   tn.z + (int64_t)b * T * C + chg, C, T, j, a.p0, a.reset_every, Aj, Bj);
        accB = accA * Bj + accB;
        accA *= Aj;
        if (j == 0) {
          const int hh = chg / a.Dh;
          const float h0v = tn.h0 ? tn.h0[((int64_t)b * a.H + hh) * a.Dh + (chg - hh * a.Dh)] : 0.f;
          carry = accA * h0v + accB;
          done = true;
        }
        --j;
        spins = 0;
      } else {
        __builtin_amdgcn_s_sleep(2);
      }
    }
  }
  return carry;
}

template <typename XT, int NC, bool RESET>
__global__ __launch_bounds__(kNW * 64) void scan_kernel(const ScanArgs a) {
  using V = XVec<XT, NC>;
  using Z = XVec<float, NC>;
  constexpr int SC = 64 * NC;   // channels per slab
  static_assert(SC <= kNW * 64, "one look-back thread per channel");
  __shared__ float s_A[kNW][SC];
  __shared__ float s_B[kNW][SC];
  __shared__ float s_carry[kNW][SC];
  // transposed-output staging: [channel][step] of this chunk (bf16 path)
  constexpr int kTRow = kChunkT * 2 + 16;   // bytes per channel row (padded)
  __shared__ __attribute__((aligned(16))) char s_T[sizeof(XT) == 2 ? SC * kTRow : 16];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const uint32_t ticket = blockIdx.x;
  const uint32_t epoch = a.hdr[1];
  // polls of an unpublished predecessor before its aggregate is computed
  // locally: the workspace header's poll_limit (n > 0: n - 1), else the default
  const uint32_t poll_word = a.hdr[3];
  const uint32_t fallback_spins = poll_word ? poll_word - 1u : kFallbackSpins;

  const int chunk = int(ticket / uint32_t(a.n_slabs));
  const int slab = int(ticket - uint32_t(chunk) * uint32_t(a.n_slabs));
  const int per_tensor = a.B * a.slabs_per_bt;
  const int ti = slab / per_tensor;
  const int rem = slab - ti * per_tensor;
  const int b = rem / a.slabs_per_bt;
  const int cs = rem - b * a.slabs_per_bt;
  const ScanTensor tn = ti == 0 ? a.ten[0] : a.ten[1];
  const int64_t C = a.C;
  const int T = a.T;
  const int t0 = chunk * kChunkT + wave * kLW;
  const int ch = cs * SC + lane * NC;   // first channel of this lane in [0, C)
  const int h = ch / a.Dh;
  const int d = ch - h * a.Dh;

  // wave-uniform row bases (scalar) plus a small per-lane offset
  const XT* xbase = static_cast<const XT*>(tn.x) + (int64_t)b * T * C + cs * SC;
  const float* zbase = tn.z + (int64_t)b * T * C + cs * SC;
  const int lo = lane * NC;

  // ---- load this wave's kLW steps (every element is read exactly once, as
  // a stream: non-temporal).  Rows past T read row T-1, which the passes
  // leave out: no branch around a load, so that no arithmetic lands between
  // the loads with a wait for each.
  typename V::raw xr[kLW];
  typename Z::raw zr[kLW];
#pragma unroll
  for (int s = 0; s < kLW; ++s) {
    const int t = min(t0 + s, T - 1);
    xr[s] = V::load_nt(xbase + (int64_t)t * C + lo);
    zr[s] = Z::load_nt(zbase + (int64_t)t * C + lo);
  }

  // first restart position >= p0 + t0 (chunk-local recurrence), or none
  // (kept relative to input row 0, as a 32-bit row index; INT_MAX: none)
  int first_reset = 0x7fffffff;
  if (a.reset_every > 0) {
    const int64_t ja = a.p0 + t0;
    first_reset = int(min<int64_t>((ja + a.reset_every - 1) / a.reset_every * a.reset_every - a.p0, 0x7fffffff));
  }

  // ---- pass 1: aggregate of the wave's steps (identity past the end)
  {
    float hl[NC], pp[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) { hl[c] = 0.f; pp[c] = 1.f; }
    int next_reset = first_reset;
#pragma unroll
    for (int s = 0; s < kLW; ++s) {
      const bool live = (t0 + s) < T;
      const bool rs = RESET && t0 + s == next_reset;
      if (rs) next_reset = sat_add(next_reset, a.reset_every);
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const float cc = gate_comp(Z::get(zr[s], c));
        Z::set(zr[s], c, cc);   // pass 2 reads 1 - g from here
        const float xv = V::get(xr[s], c);
        const float hn = rs ? cc * xv : fmaf(cc, xv, fmaf(-cc, hl[c], hl[c]));   // (1 - c) h + c x
        const float pn = rs ? 0.f : fmaf(-pp[c], cc, pp[c]);                     // (1 - c) p
        hl[c] = live ? hn : hl[c];   // a step past T (a repeated row) leaves the aggregate alone
        pp[c] = live ? pn : pp[c];
      }
    }
#pragma unroll
    for (int c = 0; c < NC; ++c) { s_A[wave][lane * NC + c] = pp[c]; s_B[wave][lane * NC + c] = hl[c]; }
  }
  __syncthreads();

  // ---- one thread per channel: chunk aggregate, look-back, per-wave carries
  if (tid < SC) {
    const int cl = tid;   // channel within the slab
    float A = 1.f, Bv = 0.f;
#pragma unroll
    for (int w = 0; w < kNW; ++w) {
      const float Aw = s_A[w][cl];
      Bv = Aw * Bv + s_B[w][cl];
      A *= Aw;
    }
    const int64_t widx = (int64_t)ticket * SC + cl;
    const float carry = chunk_carry<XT, RESET, SC>(a, tn, ticket, chunk, slab, b, cs, cl, A, Bv, epoch, fallback_spins);
    publish(a.incl + widx, tag_word(A * carry + Bv, epoch));
    float cw = carry;
#pragma unroll
    for (int w = 0; w < kNW; ++w) {
      s_carry[w][cl] = cw;
      cw = s_A[w][cl] * cw + s_B[w][cl];
    }
  }
  __syncthreads();

  // ---- pass 2: the recurrence from the carry-in (1 - g kept from pass 1);
  // stores.  The registers are hidden from the optimiser so that it does not
  // keep pass 1's gates alive across the look-back instead.
#pragma unroll
  for (int s = 0; s < kLW; ++s) { V::hide(xr[s]); Z::hide(zr[s]); }
  float hv[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) hv[c] = s_carry[wave][lane * NC + c];

  const int D = tn.grid_mode == kGridToken ? a.heads.dil[0] : a.heads.dil[h];
  // first grid position >= p0 + t0 (absolute): smallest j with (j + 1) % D == 0
  const int64_t ja0 = a.p0 + t0;
  int64_t next_grid_abs = (ja0 / D) * D + (D - 1);
  if (next_grid_abs < ja0) next_grid_abs += D;
  // row index (relative to input row 0) of the next grid state and its entry
  int next_grid = int(min<int64_t>(next_grid_abs - a.p0, 0x7fffffff));
  int64_t grid_i = (next_grid_abs + 1) / D - 1;

  XT* out_all = static_cast<XT*>(tn.out_all);
  // a head with no stored grid (capacity 0 in a per-head layout) reads its
  // grid entries from the all-state outputs instead
  XT* out_grid = tn.grid_mode != kGridToken && a.heads.gcap[h] == 0 ? nullptr
                                                                   : static_cast<XT*>(tn.out_grid);
  const int64_t G_tok = T / D;
  const bool tok_all = out_all && tn.all_mode == kAllToken;
  const bool col_all = out_all && tn.all_mode == kAllHeadCol;
  const bool col_grid = out_grid && tn.grid_mode == kGridHeadCol;
  // A dense head's transposed grid (D = 1, entry i at position i, chunks
  // 64-aligned) takes the LDS-staged 16-byte stores of the all-state output;
  // stage_grid (block-uniform) says whether any head of the slab does so.
  bool stage_grid = false;
  if (sizeof(XT) == 2 && tn.out_grid && tn.grid_mode == kGridHeadCol && (a.p0 & 63) == 0) {
    for (int hh = cs * SC / a.Dh; hh <= (cs * SC + SC - 1) / a.Dh; ++hh)
      stage_grid |= a.heads.dil[hh] == 1 && a.heads.gcap[hh] > 0 && (a.heads.gcap[hh] & 63) == 0;
  }
  const bool dense_col = stage_grid && col_grid && D == 1 && (a.heads.gcap[h] & 63) == 0;
  // A head with 2 <= D <= kSparseMaxD (a chunk holds 128 / D >= 4 of its
  // grid entries) takes them from the same staging after the chunk: a
  // (channel, 4-entry group) task stores four entries that are contiguous in
  // col_key_pos order as one 8-byte piece, or at the chunk's edges its own
  // entries one by one, instead of 2-byte stores to 64 rows per instruction.
  // stage_sparse (block-uniform): some head of the slab does so.
  bool stage_sparse = false;
  if (sizeof(XT) == 2 && tn.out_grid && tn.grid_mode == kGridHeadCol) {
    for (int hh = cs * SC / a.Dh; hh <= (cs * SC + SC - 1) / a.Dh; ++hh)
      stage_sparse |= a.heads.dil[hh] > 1 && a.heads.dil[hh] <= kSparseMaxD && a.heads.gcap[hh] > 0;
  }
  const bool sparse_col = stage_sparse && col_grid && D > 1 && D <= kSparseMaxD;
  // per-channel row bases of the column layouts
  const int64_t col_all_row = (((int64_t)b * a.H + h) * a.Dh + d) * a.tpad;
  const int64_t col_grid_row = col_grid ? grid_row_offset(a.heads, a.B, b, h, 0, a.Dh) +
                                              (int64_t)d * a.heads.gcap[h] : 0;
  float run[NC][4];
  int next_reset = first_reset;

#pragma unroll
  for (int s = 0; s < kLW; ++s) {
    const int t = t0 + s;
    const bool rs = RESET && t == next_reset;
    if (rs) next_reset = sat_add(next_reset, a.reset_every);
    if (t < T) {
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const float cc = Z::get(zr[s], c);
        const float xv = V::get(xr[s], c);
        // (1 - c) h + c x; at a chunk start the state restarts from zero
        hv[c] = rs ? cc * xv : fmaf(cc, xv, fmaf(-cc, hv[c], hv[c]));
      }
      if (tok_all) V::store(out_all + ((int64_t)b * a.arows + a.all_row0 + t) * C + cs * SC + lo, hv);
      if (out_grid && t == next_grid) {
        const int64_t i = grid_i++;
        if (tn.grid_mode == kGridToken) {
          V::store(out_grid + (((int64_t)b * G_tok + i) * a.H + h) * a.Dh + d, hv);
        } else if (tn.grid_mode == kGridHeadRow) {
          V::store(out_grid + grid_row_offset(a.heads, a.B, b, h, i, a.Dh) + d, hv);
        } else if (!dense_col && !sparse_col) {
#pragma unroll
          for (int c = 0; c < NC; ++c)
            store1(out_grid + col_grid_row + (int64_t)c * a.heads.gcap[h] + col_key_pos(i, d + c), hv[c]);
        }
        next_grid = sat_add(next_grid, D);
      }
      if (tn.h_last && t == T - 1) {
#pragma unroll
        for (int c = 0; c < NC; ++c) tn.h_last[((int64_t)b * a.H + h) * a.Dh + d + c] = hv[c];
      }
    }
    if (col_all || dense_col || sparse_col) {
      // keys t-3..t of each channel; positions past T are written as zeros
#pragma unroll
      for (int c = 0; c < NC; ++c) run[c][s & 3] = t < T ? hv[c] : 0.f;
      if ((s & 3) == 3) {
        if constexpr (sizeof(XT) == 2) {
          // stage in LDS; written out row by row below
#pragma unroll
          for (int c = 0; c < NC; ++c)
            store4(reinterpret_cast<bf16_t*>(s_T + (lane * NC + c) * kTRow) + wave * kLW + (s - 3), run[c]);
        } else if (a.all_row0 + t - 3 < a.tpad) {
#pragma unroll
          for (int c = 0; c < NC; ++c)
            store4(out_all + col_all_row + (int64_t)c * a.tpad + col_key_pos(a.all_row0 + t - 3, d + c), run[c]);
        }
      }
    }
  }
  if constexpr (sizeof(XT) == 2) {
    if (col_all || stage_grid || stage_sparse) {
      // Write the chunk's [channel][128 keys] block into the transposed rows
      // with 16-byte stores.  In col_key_pos order the physical 8-key chunk p
      // of a 64-key tile holds logical chunk c = p ^ col_swz(d): keys
      // 16(c/2) + 4(c%2) + {0..3} and the four keys 8 further on.
      __syncthreads();
      const int64_t key0 = a.all_row0 + (int64_t)chunk * kChunkT;   // a multiple of 64
      const int64_t gkey0 = a.p0 + (int64_t)chunk * kChunkT;       // dense grid entry of step 0
      constexpr int CPR = kChunkT / 8;   // 16-byte chunks per channel row
#pragma unroll
      for (int k = 0; k < SC * CPR / (kNW * 64); ++k) {
        const int task = tid + kNW * 64 * k;
        const int r = task / CPR;          // channel within the slab
        const int p = task - r * CPR;      // physical chunk within the 128 keys
        const int chg = cs * SC + r;
        const int hh = chg / a.Dh;
        const int dd = chg - hh * a.Dh;
        const int lc = (p & 7) ^ col_swz(dd);
        const int k0 = 64 * (p >> 3) + 16 * (lc >> 1) + 4 * (lc & 1);   // first key, natural order
        const uint2 w0 = *reinterpret_cast<const uint2*>(s_T + r * kTRow + 2 * k0);
        const uint2 w1 = *reinterpret_cast<const uint2*>(s_T + r * kTRow + 2 * (k0 + 8));
        const uint4 w = make_uint4(w0.x, w0.y, w1.x, w1.y);
        const int64_t kpos = key0 + p * 8;
        if (col_all && kpos < a.tpad)
          *reinterpret_cast<uint4*>(out_all + (((int64_t)b * a.H + hh) * a.Dh + dd) * a.tpad + kpos) = w;
        const int gc = a.heads.gcap[hh];
        const int64_t gpos = gkey0 + p * 8;
        if (stage_grid && a.heads.dil[hh] == 1 && gc > 0 && (gc & 63) == 0 && gpos < gc)
          *reinterpret_cast<uint4*>(static_cast<XT*>(tn.out_grid) + grid_row_offset(a.heads, a.B, b, hh, 0, a.Dh) +
                                    (int64_t)dd * gc + gpos) = w;
      }
      if (stage_sparse) {
        // grid entries i whose positions (i + 1) D - 1 lie in the chunk's
        // [pa, pb): i in [ia, ib), in groups of four from ia rounded down;
        // per head of the slab (one or two: Dh is 64 or 128) its first entry,
        // group count and D, then one task per (group, channel)
        const int pa = int(a.p0) + chunk * kChunkT;
        const int pb = int(a.p0) + min((chunk + 1) * kChunkT, T);
        const int dsh = 31 - __builtin_clz(a.Dh);        // log2(Dh)
        const int h_lo = (cs * SC) >> dsh;
        int ia2[2], nq2[2], dg2[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int hh = h_lo + j;
          const bool in = hh <= ((cs * SC + SC - 1) >> dsh);
          const int Dg = in ? a.heads.dil[hh] : 0;
          const bool use = in && Dg > 1 && Dg <= kSparseMaxD && a.heads.gcap[hh] > 0;
          const int ia = use ? (pa + Dg) / Dg - 1 : 0, ib = use ? (pb + Dg) / Dg - 1 : 0;
          ia2[j] = ia;
          nq2[j] = use && ib > ia ? ((ib - 1) >> 2) - (ia >> 2) + 1 : 0;
          dg2[j] = Dg;
        }
        const int G = max(nq2[0], nq2[1]);
        for (int task = tid; task < SC * G; task += kNW * 64) {
          const int q = task / SC, r = task - q * SC;     // SC is a power of two
          const int chg = cs * SC + r;
          const int j = (chg >> dsh) - h_lo;
          const int dd = chg & (a.Dh - 1);
          const int Dg = j ? dg2[1] : dg2[0];
          const int ia = j ? ia2[1] : ia2[0];
          if (q >= (j ? nq2[1] : nq2[0])) continue;
          const int ib = (pb + Dg) / Dg - 1;
          const int g0 = (ia & ~3) + 4 * q;
          const int hh = h_lo + j;
          const int gc = a.heads.gcap[hh];
          const uint16_t* row = reinterpret_cast<const uint16_t*>(s_T + r * kTRow);
          uint16_t* dst = reinterpret_cast<uint16_t*>(static_cast<XT*>(tn.out_grid) +
                                                      grid_row_offset(a.heads, a.B, b, hh, 0, a.Dh) + (int64_t)dd * gc);
          if (g0 >= ia && g0 + 4 <= ib) {
            uint32_t v[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = row[(g0 + e + 1) * Dg - 1 - pa];
            *reinterpret_cast<uint2*>(dst + col_key_pos(g0, dd)) = make_uint2(v[0] | (v[1] << 16), v[2] | (v[3] << 16));
          } else {
            for (int i = max(g0, ia); i < min(g0 + 4, ib); ++i) dst[col_key_pos(i, dd)] = row[(i + 1) * Dg - 1 - pa];
          }
        }
      }
    }
  }
  // the wave holding position T-1 zero-fills the column grid past its last entry
  if (col_grid && t0 <= T - 1 && T - 1 < t0 + kLW) {
    const int cap = a.heads.gcap[h];
    for (int64_t i = (a.p0 + T) / D; i < cap; ++i) {
#pragma unroll
      for (int c = 0; c < NC; ++c)
        store1(out_grid + col_grid_row + (int64_t)c * cap + col_key_pos(i, d + c), 0.f);
    }
  }
}

// Segmented scan for grid-only outputs (no all-state output, no restart,
// every stored grid with D >= kLW, so a wave's kLW steps hold at most one
// grid position).  Block = (segment, slab), kSegNW waves, one block per CU:
// a contiguous run of seg_chunks chunks of kSegChunkT steps of one slab,
// walked in order with the next chunk's inputs in flight while the current
// one is folded.  (Two 8-wave blocks per CU ran unevenly: the older block's
// waves win the issue arbitration, and the younger block set the kernel's
// time at ~1.33x the older one's.)  Phase A: per chunk, each wave folds its
// steps into its aggregate and the partial aggregate up to its grid
// position; one thread per channel keeps the segment's running aggregate and
// hands every wave the aggregate from the segment start to the wave's first
// step, so each grid position gets its (A, B) relative to the segment start,
// written to part[] (state = A * carry_in + B).  The segment's aggregate then
// goes through the same decoupled look-back as the chunked scan, over
// segments instead of chunks (a handful per slab, all resident at once), and
// phase B turns the pairs into grid states with one FMA each.  Every input
// element is read once; part[] adds 8 bytes per grid element written and
// read.
template <typename XT, int NC>
__global__ __launch_bounds__(kSegNW * 64) void scan_seg_kernel(const ScanArgs a) {
  using V = XVec<XT, NC>;
  using Z = XVec<float, NC>;
  constexpr int SC = 64 * NC;   // channels per slab
  static_assert(SC <= kSegNW * 64, "one prefix thread per channel");
  __shared__ float s_A[kSegNW][SC];
  __shared__ float s_B[kSegNW][SC];
  __shared__ float s_PA[kSegNW][SC];   // aggregate from the segment start to each wave's first step
  __shared__ float s_PB[kSegNW][SC];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const uint32_t epoch = a.hdr[1];
  const uint32_t poll_word = a.hdr[3];
  // segments publish about together; a wait this long means a segment that
  // is not running (the device is shared), whose aggregate is then computed
  // here from its inputs
  const uint32_t fallback_spins = poll_word ? poll_word - 1u : kFallbackSpins * 256u;
  const int64_t C = a.C;
  const int T = a.T;
  const int n_chunks = int(((int64_t)T + kSegChunkT - 1) / kSegChunkT);
  const int seg = int(blockIdx.x) / a.n_slabs;
  const int slab = int(blockIdx.x) - seg * a.n_slabs;
  const int per_tensor = a.B * a.slabs_per_bt;
  const int ti = slab / per_tensor;
  const int rem = slab - ti * per_tensor;
  const int b = rem / a.slabs_per_bt;
  const int cs = rem - b * a.slabs_per_bt;
  const ScanTensor tn = ti == 0 ? a.ten[0] : a.ten[1];
  float* const part = ti == 0 ? a.part[0] : a.part[1];
  const int lo = lane * NC;
  const int ch = cs * SC + lo;   // first channel of this lane in [0, C)
  const int h = ch / a.Dh;
  const int d = ch - h * a.Dh;
  const int D = tn.grid_mode == kGridToken ? a.heads.dil[0] : a.heads.dil[h];
  const int c_begin = seg * a.seg_chunks;
  const int c_end = min(n_chunks, c_begin + a.seg_chunks);
  const int64_t G_tok = T / D;
  // per-lane table lookups taken once (inside the loops a memory clobber
  // would reload them, and a vector load there waits for the inputs in flight)
  const int gcap = a.heads.gcap[h];
  XT* const out_grid = tn.grid_mode != kGridToken && gcap == 0 ? nullptr : static_cast<XT*>(tn.out_grid);
  const int64_t grow0 = tn.grid_mode == kGridToken ? 0 : grid_row_offset(a.heads, a.B, b, h, 0, a.Dh);
  // element index of grid entry i of this lane's first channel (row-major)
  auto grid_elem = [&](int64_t i) __attribute__((always_inline)) -> int64_t {
    return tn.grid_mode == kGridToken ? (((int64_t)b * G_tok + i) * a.H + h) * a.Dh + d
                                      : grow0 + i * a.Dh + d;
  };
  // the same entry's (A, B) pair in part[]: head-major in both layouts, so
  // that a block's pairs fill one run of memory in entry order
  auto part_elem = [&](int64_t i) __attribute__((always_inline)) -> int64_t {
    return tn.grid_mode == kGridToken ? (((int64_t)b * a.H + h) * G_tok + i) * a.Dh + d
                                      : grow0 + i * a.Dh + d;
  };
  // The next grid position at or after this wave's first step in phase A,
  // tracked from chunk to chunk without divisions: r = its offset from the
  // first step (in [0, D)), pe = its entry's pair index in part[].  A chunk
  // moves the first step kSegChunkT = mq * D + mr rows on.
  const int mq = kSegChunkT / D, mr = kSegChunkT - mq * D;
  int r;
  int64_t pe;
  {
    const int64_t ja0 = a.p0 + (int64_t)c_begin * kSegChunkT + wave * kLW;
    int64_t nxt = (ja0 / D) * D + (D - 1);
    if (nxt < ja0) nxt += D;
    r = int(nxt - ja0);
    pe = part_elem((nxt + 1) / D - 1);
  }
  auto advance = [&]() __attribute__((always_inline)) {
    r -= mr;
    const bool wrap = r < 0;
    r += wrap ? D : 0;
    pe += (int64_t)(mq + (wrap ? 1 : 0)) * a.Dh;
  };

  const XT* xbase = static_cast<const XT*>(tn.x) + (int64_t)b * T * C + cs * SC;
  const float* zbase = tn.z + (int64_t)b * T * C + cs * SC;
  typename V::raw xr[kLW];
  typename Z::raw zr[kLW];
  // step s of this wave's kLW steps from row t0.  Rows past T read row T-1
  // (what phase A folds in from them reaches no stored value): no branch
  // around the loads, so the compiler's wait counts stay exact and the loads
  // of the next chunk stay in flight under the current one.
  // The inputs are read once, as a stream: non-temporal loads, which keep
  // them from displacing the (A, B) pairs from the caches on their way to
  // memory (with plain loads the scan runs ~9% slower on T = 262144).
  auto load_step = [&](int t0, int s) __attribute__((always_inline)) {
    const int t = min(t0 + s, T - 1);
    xr[s] = V::load_nt(xbase + (int64_t)t * C + lo);
    zr[s] = Z::load_nt(zbase + (int64_t)t * C + lo);
  };

  // ---- phase A
  float segA = 1.f, segB = 0.f;            // prefix thread: the segment's running aggregate
  float lA[NC], lB[NC];                    // the lane holding T-1: its aggregate from the segment start
#pragma unroll
  for (int c = 0; c < NC; ++c) { lA[c] = 1.f; lB[c] = 0.f; }
  // the first chunk's rows in step order, as the loop reloads them (the wait
  // for step 0 at the loop head is taken over both entries to the loop: out
  // of order here, it would wait for the whole chunk on every iteration)
#pragma unroll
  for (int s = 0; s < kLW; ++s) {
    load_step(c_begin * kSegChunkT + wave * kLW, s);
    asm volatile("" ::: "memory");
  }
  for (int c = c_begin; c < c_end; ++c) {
    const int t0 = c * kSegChunkT + wave * kLW;
    // rows of the next chunk, loaded step by step into the registers pass 1
    // has just consumed, so that a chunk's worth of loads is always in
    // flight (past the segment's last chunk: rows past T, nothing read)
    const int t0n = (c + 1 < c_end ? c + 1 : n_chunks) * kSegChunkT + wave * kLW;
    const int gs = (out_grid && r < kLW && t0 + r < T) ? r : -1;
    const int ls = (tn.h_last && t0 <= T - 1 && T - 1 < t0 + kLW) ? T - 1 - t0 : -1;   // uniform
    float hl[NC], pp[NC], gA[NC], gB[NC], qA[NC], qB[NC];
#pragma unroll
    for (int k = 0; k < NC; ++k) { hl[k] = 0.f; pp[k] = 1.f; gA[k] = qA[k] = 1.f; gB[k] = qB[k] = 0.f; }
    V::hide(xr[0]);
    Z::hide(zr[0]);
#pragma unroll
    for (int s = 0; s < kLW; ++s) {
      // Steps past T (repeated rows in the last chunk) are folded in too:
      // what follows T-1 reaches no stored value (no grid position or h_last
      // lies past it, and no later segment or wave reads the aggregates).
#pragma unroll
      for (int k = 0; k < NC; ++k) {
        const float cc = gate_comp(Z::get(zr[s], k));
        hl[k] = fmaf(cc, V::get(xr[s], k), fmaf(-cc, hl[k], hl[k]));   // (1 - c) h + c x
        pp[k] = fmaf(-pp[k], cc, pp[k]);                                 // (1 - c) p
        gA[k] = s == gs ? pp[k] : gA[k];
        gB[k] = s == gs ? hl[k] : gB[k];
        // taken here, step by step (else every step's products stay live
        // for a selection at the end)
        opaque(gA[k]); opaque(gB[k]);
      }
      if (s == ls) {
#pragma unroll
        for (int k = 0; k < NC; ++k) { qA[k] = pp[k]; qB[k] = hl[k]; }
      }
      asm volatile("" ::: "memory");   // the reload stays after this step's use
      load_step(t0n, s);
      // step s + 1 is used only from here on (else the compiler hoists its
      // arithmetic above the reloads and waits for the whole chunk at once)
      if (s + 1 < kLW) {
        V::hide(xr[s + 1]);
        Z::hide(zr[s + 1]);
      }
    }
#pragma unroll
    for (int k = 0; k < NC; ++k) { s_A[wave][lo + k] = pp[k]; s_B[wave][lo + k] = hl[k]; }
    __syncthreads();
    if (tid < SC) {
      float pA = segA, pB = segB;
#pragma unroll
      for (int w = 0; w < kSegNW; ++w) {
        s_PA[w][tid] = pA;
        s_PB[w][tid] = pB;
        const float Aw = s_A[w][tid];
        pB = Aw * pB + s_B[w][tid];
        pA *= Aw;
      }
      segA = pA;
      segB = pB;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < NC; ++k) {
      const float PA = s_PA[wave][lo + k], PB = s_PB[wave][lo + k];
      if (gs >= 0)
        *reinterpret_cast<float2*>(part + 2 * (pe + k)) = make_float2(gA[k] * PA, gA[k] * PB + gB[k]);
      if (ls >= 0) { lA[k] = qA[k] * PA; lB[k] = qA[k] * PB + qB[k]; }
    }
    advance();
  }

  // ---- the segment's carry-in: look-back over earlier segments of the slab
  __shared__ float s_cin[SC];
  if (tid < SC) {
    const int cl = tid;
    const int64_t widx = ((int64_t)seg * a.n_slabs + slab) * SC + cl;
    float carry = 0.f;
    if (seg == 0) {
      const int chg = cs * SC + cl;
      const int hh = chg / a.Dh;
      carry = tn.h0 ? tn.h0[((int64_t)b * a.H + hh) * a.Dh + (chg - hh * a.Dh)] : 0.f;
    } else {
      publish(a.agg_a + widx, tag_word(segA, epoch));
      publish(a.agg_b + widx, tag_word(segB, epoch));
      float accA = 1.f, accB = 0.f;
      int j = seg - 1;
      uint32_t spins = 0;
      bool done = false;
      while (!done) {
        const int64_t pidx = ((int64_t)j * a.n_slabs + slab) * SC + cl;
        const uint64_t wi = peek(a.incl + pidx);
        const uint64_t wa = peek(a.agg_a + pidx);
        const uint64_t wb = peek(a.agg_b + pidx);
        if (uint32_t(wi >> 32) == epoch) {
          carry = accA * word_value(wi) + accB;
          done = true;
        } else if (uint32_t(wa >> 32) == epoch && uint32_t(wb >> 32) == epoch) {
          accB = accA * word_value(wb) + accB;
          accA *= word_value(wa);
          --j;
          spins = 0;
        } else if (++spins > fallback_spins) {
          // segment j shows no progress: fold its chunks in from the inputs
          const int chg = cs * SC + cl;
          float Aj = 1.f, Bj = 0.f;
          constexpr int per = kSegChunkT / kChunkT;   // plain chunks per segment chunk
          const int nc_plain = int(((int64_t)T + kChunkT - 1) / kChunkT);
          for (int cj = j * a.seg_chunks * per; cj < min(nc_plain, (j + 1) * a.seg_chunks * per); ++cj) {
            float Ac, Bc;
            chunk_aggregate<XT, false>(static_cast<const XT*>(tn.x) + (int64_t)b * T * C + chg,
                                       tn.z + (int64_t)b * T * C + chg, C, T, cj, a.p0, 0, Ac, Bc);
            Bj = Ac * Bj + Bc;
            Aj *= Ac;
          }
          accB = accA * Bj + accB;
          accA *= Aj;
          if (j == 0) {
            const int hh = chg / a.Dh;
            const float h0v = tn.h0 ? tn.h0[((int64_t)b * a.H + hh) * a.Dh + (chg - hh * a.Dh)] : 0.f;
            carry = accA * h0v + accB;
            done = true;
          }
          --j;
          spins = 0;
        } else {
          __builtin_amdgcn_s_sleep(2);
        }
      }
    }
    publish(a.incl + widx, tag_word(segA * carry + segB, epoch));
    s_cin[cl] = carry;
  }
  __syncthreads();

  // ---- phase B: grid states (and h_last) from the carry-in
  float cin[NC];
#pragma unroll
  for (int k = 0; k < NC; ++k) cin[k] = s_cin[lo + k];
  // The segment's entries are spread over the waves, kPB of them in flight
  // per lane (each is a load, an FMA and a store).
  if (out_grid) {
    constexpr int kPB = 4;
    const int64_t pos_lo = a.p0 + (int64_t)c_begin * kSegChunkT;
    const int64_t pos_hi = a.p0 + min((int64_t)c_end * kSegChunkT, (int64_t)T);
    const int64_t e_lo = (pos_lo + D) / D - 1;   // first entry at or after pos_lo
    const int64_t e_hi = pos_hi / D;             // entries before pos_hi
    const int64_t pe_lo = part_elem(e_lo);
    for (int64_t e0 = e_lo + wave; e0 < e_hi; e0 += kSegNW * kPB) {
      float2 ab[kPB][NC];
#pragma unroll
      for (int j = 0; j < kPB; ++j) {
        const int64_t e = min(e0 + j * kSegNW, e_hi - 1);
        const int64_t q = pe_lo + (e - e_lo) * a.Dh;
#pragma unroll
        for (int k = 0; k < NC; ++k) ab[j][k] = *reinterpret_cast<const float2*>(part + 2 * (q + k));
      }
#pragma unroll
      for (int j = 0; j < kPB; ++j) {
        const int64_t e = e0 + j * kSegNW;
        if (e >= e_hi) break;
        float hv[NC];
#pragma unroll
        for (int k = 0; k < NC; ++k) hv[k] = ab[j][k].x * cin[k] + ab[j][k].y;
        if (tn.grid_mode == kGridHeadCol) {
          const int64_t row = grow0 + (int64_t)d * gcap;
#pragma unroll
          for (int k = 0; k < NC; ++k) store1(out_grid + row + (int64_t)k * gcap + col_key_pos(e, d + k), hv[k]);
        } else {
          V::store(out_grid + grid_elem(e), hv);
        }
      }
    }
  }
  // the wave holding position T-1
  if (c_end == n_chunks && wave == ((T - 1) % kSegChunkT) / kLW) {
    if (tn.h_last) {
#pragma unroll
      for (int k = 0; k < NC; ++k) tn.h_last[((int64_t)b * a.H + h) * a.Dh + d + k] = lA[k] * cin[k] + lB[k];
    }
    // the column grid past its last entry is zero
    if (out_grid && tn.grid_mode == kGridHeadCol) {
      const int cap = gcap;
      const int64_t row = grow0 + (int64_t)d * cap;
      for (int64_t i = (a.p0 + T) / D; i < cap; ++i) {
#pragma unroll
        for (int k = 0; k < NC; ++k) store1(out_grid + row + (int64_t)k * cap + col_key_pos(i, d + k), 0.f);
      }
    }
  }
}

// Blocks of `fn` (`threads` each) that fit on the current device at once.
int resident_blocks(const void* fn, int threads) {
  int dev = 0, cus = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, threads, 0) != hipSuccess)
    return 0;
  return cus * per_cu;
}

// Grid states only: no tensor stores every state, no restart, every stored
// grid has D >= kLW.
bool grid_only(const ScanTensor* ten, int ntensors, int reset_every, int H, const HeadTable& heads) {
  if (reset_every > 0) return false;
  for (int t = 0; t < ntensors; ++t) {
    if (ten[t].out_all) return false;
    if (!ten[t].out_grid) continue;
    if (ten[t].grid_mode == kGridToken) {
      if (heads.dil[0] < kLW) return false;
    } else {
      for (int h = 0; h < H; ++h)
        if (heads.gcap[h] > 0 && heads.dil[h] < kLW) return false;
    }
  }
  return true;
}

// Segments per slab: as many as fill the device once with every slab's
// segments resident together, each at least one chunk.
template <typename XT, int NC>
hipError_t launch_segmented(ScanArgs a, hipStream_t s) {
  const int resident = resident_blocks(reinterpret_cast<const void*>(&scan_seg_kernel<XT, NC>), kSegNW * 64);
  if (resident <= 0) return hipErrorInvalidDevice;
  const int n_chunks = int(((int64_t)a.T + kSegChunkT - 1) / kSegChunkT);
  int n_seg = resident / a.n_slabs;
  n_seg = n_seg < 1 ? 1 : n_seg > n_chunks ? n_chunks : n_seg;
  a.seg_chunks = (n_chunks + n_seg - 1) / n_seg;
  a.n_seg = (n_chunks + a.seg_chunks - 1) / a.seg_chunks;   // no empty segment
  hipLaunchKernelGGL((scan_seg_kernel<XT, NC>), dim3(a.n_seg * a.n_slabs), dim3(kSegNW * 64), 0, s, a);
  return hipGetLastError();
}

template <typename XT, int NC>
hipError_t launch_typed(const ScanArgs& a, int n_chunks, hipStream_t s) {
  const int blocks = n_chunks * a.n_slabs;
  // the chunk-local restart is a separate instantiation: the plain scan
  // carries no per-step check for it
  if (a.reset_every > 0)
    hipLaunchKernelGGL((scan_kernel<XT, NC, true>), dim3(blocks), dim3(kNW * 64), 0, s, a);
  else
    hipLaunchKernelGGL((scan_kernel<XT, NC, false>), dim3(blocks), dim3(kNW * 64), 0, s, a);
  return hipGetLastError();
}

// Channels per lane.  Two (128-channel slabs) measured best on MI355X: twice
// as many independent carry chains as four, each with half the chunks in
// flight, at equal coalescing (256-byte rows of x per wave load).
int pick_nc(int C) {
  if (C % 128 == 0) return 2;
  return 1;
}

}  // namespace

bool scan_grid_only(const ScanPlan& p) { return grid_only(p.ten, p.ntensors, p.reset_every, p.H, p.heads); }

size_t scan_workspace_bytes(int ntensors, int B, int T, int H, int Dh) {
  const int64_t C = (int64_t)H * Dh;
  const int64_t n_chunks = (T + kChunkT - 1) / kChunkT;
  const int64_t words = n_chunks * ntensors * (int64_t)B * C;   // one word per (chunk, channel)
  return sizeof(WsHeader) + 3 * (size_t)words * sizeof(uint64_t);
}

hipError_t launch_scan(const ScanPlan& p, hipStream_t s) {
  if (p.T <= 0 || p.B <= 0) return hipSuccess;
  ScanArgs a;
  a.part[0] = a.part[1] = nullptr;
  a.n_seg = a.seg_chunks = 0;
  a.ten[0] = p.ten[0];
  a.ten[1] = p.ntensors > 1 ? p.ten[1] : p.ten[0];
  a.B = p.B; a.T = p.T; a.H = p.H; a.Dh = p.Dh; a.C = p.H * p.Dh;
  a.tpad = p.tpad;
  a.p0 = p.p0;
  a.all_row0 = p.all_row0;
  a.arows = p.arows > 0 ? p.arows : p.T;
  a.reset_every = p.reset_every;
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
  if (p.part[0] && scan_grid_only(p)) {
    a.part[0] = p.part[0];
    a.part[1] = p.ntensors > 1 ? p.part[1] : p.part[0];
    if (p.bf16) return nc == 2 ? launch_segmented<bf16_t, 2>(a, s) : launch_segmented<bf16_t, 1>(a, s);
    return nc == 2 ? launch_segmented<float, 2>(a, s) : launch_segmented<float, 1>(a, s);
  }
  if (p.bf16) return nc == 2 ? launch_typed<bf16_t, 2>(a, nch, s) : launch_typed<bf16_t, 1>(a, nch, s);
  return nc == 2 ? launch_typed<float, 2>(a, nch, s) : launch_typed<float, 1>(a, nch, s);
}

}  // namespace rat
