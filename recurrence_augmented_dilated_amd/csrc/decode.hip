// One decode step of the RAT+ operator for a batch of sequences.
//
// Per (b, h) at position t = pos[b] ("RAT+: Train Dense, Infer Sparse",
// Fig. 2: the recurrence is updated one step at a time while decoding and
// attention runs over the cached states; abstract: the grid cache holds every
// D-th state, so it is D times smaller, plus an optional local window):
//   1. state <- g * state + (1 - g) * x  for keys and values (fp32 state);
//   2. if W > 0 the new state goes to ring slot t mod W;
//   3. if (t + 1) mod D == 0 it is appended as grid entry (t + 1) / D - 1;
//   4. the query attends over grid entries i < max(0, t - W + 1) / D (strictly
//      older than the window when W > 0) plus the ring slots of positions
//      max(0, t - W + 1) .. t.
//
// Work items are (b, h, split).  A split streams a contiguous range of grid
// rows; the last split of a (b, h) also owns the state update, the cache
// writes and the window keys, and takes the newly written state from LDS, so
// no item reads a row another item writes in the same step.  Inside a block
// each wave streams its share of rows, LPK = Dh/8 lanes per key (one 16-byte
// bf16 load per lane per row), with a private online softmax per key slot
// and DPP reductions for the dot products; waves merge in LDS.  Items with
// several splits write (m, l, acc) partials, one slot per work item, that a
// second kernel merges in a fixed order.  Heads are launched heaviest first (per-head dilation).
#include "rat_internal.h"
#include "kv_stream.h"

namespace rat {
namespace {

constexpr int kWaves = 4;
constexpr int kUnroll = 4;

struct DecArgs {
  const void* q; const void* k; const void* v;
  const float* zk; const float* zv;
  float* state_k; float* state_v;
  void* grid_k; void* grid_v;
  void* ring_k; void* ring_v;
  const int32_t* pos;
  int64_t max_pos;
  void* out;
  float* partials;
  uint32_t* hdr;
  int B, H, W;
  float sl2;
  int reset_every;
  DecodeHeads heads;
};

template <typename ET, int DH>
__global__ __launch_bounds__(kWaves * 64) void decode_kernel(const DecArgs a) {
  using R = Row8<ET>;
  constexpr int LPK = DH / 8;        // lanes per key row
  constexpr int KPW = 64 / LPK;      // keys per wave step
  __shared__ float s_newk[DH];
  __shared__ float s_newv[DH];
  __shared__ float s_m[kWaves], s_l[kWaves];
  __shared__ float s_acc[kWaves][DH];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int rg = lane / LPK;         // key slot of this lane in a wave step
  const int c = lane - rg * LPK;     // head dims 8c .. 8c+7

  // ---- item -> (h, b, split)
  const int item = blockIdx.x;
  int oi = 0;
  while (oi + 1 < a.H && a.heads.item_base[oi + 1] <= item) ++oi;
  const int h = a.heads.order[oi];
  const int ns = a.heads.nsplit[h];
  const int rem = item - a.heads.item_base[oi];
  const int b = rem / ns;
  const int s = rem - b * ns;
  const bool owner = s == ns - 1;
  const int W = a.W;
  const int D = a.heads.t.dil[h];
  const int64_t bh = (int64_t)b * a.H + h;

  const int64_t t = a.pos[b];
  const bool bad = t < 0 || t >= a.max_pos;
  if (bad && tid == 0) atomicOr(&a.hdr[2], kErrDecodePos);

  // ---- owner: state update and cache writes
  if (owner && !bad && tid < DH) {
    const int64_t idx = bh * DH + tid;
    float gk, ck, gv, cv;
    gate_pair(a.zk[idx], gk, ck);
    gate_pair(a.zv[idx], gv, cv);
    const float xk = sizeof(ET) == 2 ? bf16_to_f32(static_cast<const bf16_t*>(a.k)[idx])
                                     : static_cast<const float*>(a.k)[idx];
    const float xv = sizeof(ET) == 2 ? bf16_to_f32(static_cast<const bf16_t*>(a.v)[idx])
                                     : static_cast<const float*>(a.v)[idx];
    // chunk-local recurrence: a position that starts a chunk drops the carried state
    const bool restart = a.reset_every > 0 && t % a.reset_every == 0;
    const float sk = (restart ? 0.f : gk * a.state_k[idx]) + ck * xk;
    const float sv = (restart ? 0.f : gv * a.state_v[idx]) + cv * xv;
    a.state_k[idx] = sk;
    a.state_v[idx] = sv;
    const float rk = R::round(sk);
    const float rv = R::round(sv);
    s_newk[tid] = rk;
    s_newv[tid] = rv;
    if (W > 0) {
      const int64_t ro = (bh * W + (t % W)) * DH + tid;
      R::store1(static_cast<ET*>(a.ring_k) + ro, rk);
      R::store1(static_cast<ET*>(a.ring_v) + ro, rv);
    }
    if ((t + 1) % D == 0) {
      const int64_t go = grid_row_offset(a.heads.t, a.B, b, h, (t + 1) / D - 1, DH) + tid;
      R::store1(static_cast<ET*>(a.grid_k) + go, rk);
      R::store1(static_cast<ET*>(a.grid_v) + go, rv);
    }
  }
  __syncthreads();

  // ---- key ranges of this item
  int64_t n_g = 0, n_mem = 0;
  int n_tail = 0;
  if (!bad) {
    const int64_t x = t - W + 1;
    n_g = x > 0 ? x / D : 0;
    const bool fresh = (t + 1) % D == 0;
    n_mem = (W == 0 && fresh) ? n_g - 1 : n_g;
    n_tail = W > 0 ? (int)min<int64_t>(W, t + 1) : (fresh ? 1 : 0);
  }
  const int64_t chunk = (n_mem + ns - 1) / ns;
  const int64_t r_lo = min<int64_t>(n_mem, (int64_t)s * chunk);
  const int64_t r_hi = min<int64_t>(n_mem, r_lo + chunk);
  const int64_t per_wave = (r_hi - r_lo + kWaves - 1) / kWaves;
  const int64_t w_lo = min<int64_t>(r_hi, r_lo + wave * per_wave);
  const int64_t w_hi = min<int64_t>(r_hi, w_lo + per_wave);

  // query slice, pre-scaled to log2 units
  float q8[8];
  {
    typename R::raw qr = R::load(static_cast<const ET*>(a.q) + bh * DH + 8 * c);
    R::get(qr, q8);
#pragma unroll
    for (int i = 0; i < 8; ++i) q8[i] *= a.sl2;
  }

  Soft st;
  st.m = -INFINITY;
  st.l = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) st.acc[i] = 0.f;

  const HeadTable& ht = a.heads.t;
  const ET* gk = static_cast<const ET*>(a.grid_k) + grid_row_offset(ht, a.B, b, h, 0, DH) + 8 * c;
  const ET* gv = static_cast<const ET*>(a.grid_v) + grid_row_offset(ht, a.B, b, h, 0, DH) + 8 * c;

  // ---- stream grid rows [w_lo, w_hi)
  for (int64_t base = w_lo; base < w_hi; base += KPW * kUnroll) {
    typename R::raw kr[kUnroll], vr[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t r = base + u * KPW + rg;
      const bool ok = r < w_hi;
      kr[u] = ok ? R::load_nt(gk + r * DH) : R::zero();
      vr[u] = ok ? R::load_nt(gv + r * DH) : R::zero();
    }
    float sc[kUnroll];
    float vv[kUnroll][8];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      float kf[8];
      R::get(kr[u], kf);
      R::get(vr[u], vv[u]);
      float d0 = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) d0 = fmaf(q8[i], kf[i], d0);
      d0 = group_sum<LPK>(d0);
      sc[u] = (base + u * KPW + rg) < w_hi ? d0 : -INFINITY;
    }
    soft_update<kUnroll>(st, sc, vv);
  }

  // ---- owner: window / fresh keys (ring slots; position t from LDS)
  if (owner && n_tail > 0) {
    const int64_t p0 = t - n_tail + 1;
    for (int u0 = wave * KPW; u0 < n_tail; u0 += kWaves * KPW) {
      const int u = u0 + rg;
      const bool ok = u < n_tail;
      float kf[8], vf[1][8];
      const int64_t p = p0 + u;
      if (ok && p == t) {
#pragma unroll
        for (int i = 0; i < 8; ++i) { kf[i] = s_newk[8 * c + i]; vf[0][i] = s_newv[8 * c + i]; }
      } else if (ok) {
        const int64_t ro = (bh * W + (p % W)) * DH + 8 * c;
        R::get(R::load(static_cast<const ET*>(a.ring_k) + ro), kf);
        R::get(R::load(static_cast<const ET*>(a.ring_v) + ro), vf[0]);
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) { kf[i] = 0.f; vf[0][i] = 0.f; }
      }
      float d0 = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) d0 = fmaf(q8[i], kf[i], d0);
      d0 = group_sum<LPK>(d0);
      float sc1[1] = {ok ? d0 : -INFINITY};
      soft_update<1>(st, sc1, vf);
    }
  }

  // ---- merge key slots inside the wave (lanes with equal c)
#pragma unroll
  for (int off = LPK; off < 64; off <<= 1) {
    const float m2 = __shfl_xor(st.m, off);
    const float l2 = __shfl_xor(st.l, off);
    float a2[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) a2[i] = __shfl_xor(st.acc[i], off);
    soft_merge(st, m2, l2, a2);
  }
  if (rg == 0) {
    if (c == 0) { s_m[wave] = st.m; s_l[wave] = st.l; }
#pragma unroll
    for (int i = 0; i < 8; ++i) s_acc[wave][8 * c + i] = st.acc[i];
  }
  __syncthreads();
  if (wave == 0 && rg == 0) {
    Soft fin;
    fin.m = s_m[0];
    fin.l = s_l[0];
#pragma unroll
    for (int i = 0; i < 8; ++i) fin.acc[i] = s_acc[0][8 * c + i];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) soft_merge(fin, s_m[w], s_l[w], &s_acc[w][8 * c]);
    if (ns == 1) {
      const float inv = fin.l > 0.f ? 1.0f / fin.l : 0.f;
      float o8[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) o8[i] = fin.acc[i] * inv;
      R::store(static_cast<ET*>(a.out) + bh * DH + 8 * c, o8);
    } else {
      // partials of work item `item`: the splits of one (b, h) are adjacent
      float* pp = a.partials + (int64_t)item * (DH + 2);
#pragma unroll
      for (int i = 0; i < 8; ++i) pp[8 * c + i] = fin.acc[i];
      if (c == 0) { pp[DH] = fin.m; pp[DH + 1] = fin.l; }
    }
  }
}

template <typename ET, int DH>
__global__ __launch_bounds__(DH) void decode_combine(const DecArgs a) {
  const int bhi = blockIdx.x;
  const int h = bhi % a.H;
  const int b = bhi / a.H;
  const int ns = a.heads.nsplit[h];
  if (ns <= 1) return;
  const int d = threadIdx.x;
  // the first work item of (b, h): head h's launch rank, then b's splits
  int oi = 0;
  while (oi + 1 < a.H && a.heads.order[oi] != h) ++oi;
  const int64_t item0 = (int64_t)a.heads.item_base[oi] + (int64_t)b * ns;
  const float* pp = a.partials + item0 * (DH + 2);
  float M = -INFINITY;
  for (int s = 0; s < ns; ++s) M = fmaxf(M, pp[s * (DH + 2) + DH]);
  float L = 0.f, O = 0.f;
  if (M != -INFINITY) {
    for (int s = 0; s < ns; ++s) {
      const float f = __builtin_amdgcn_exp2f(pp[s * (DH + 2) + DH] - M);
      L += pp[s * (DH + 2) + DH + 1] * f;
      O += pp[s * (DH + 2) + d] * f;
    }
  }
  const float o = L > 0.f ? O / L : 0.f;
  Row8<ET>::store1(static_cast<ET*>(a.out) + (int64_t)bhi * DH + d, o);
}

template <typename ET, int DH>
hipError_t launch_typed(const DecArgs& a, int n_items, bool any_split, hipStream_t s) {
  hipLaunchKernelGGL((decode_kernel<ET, DH>), dim3(n_items), dim3(kWaves * 64), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !any_split) return e;
  hipLaunchKernelGGL((decode_combine<ET, DH>), dim3(a.B * a.H), dim3(DH), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const DecodePlan& p, hipStream_t s) {
  if (p.B <= 0 || p.n_items <= 0) return hipSuccess;
  DecArgs a;
  a.q = p.q; a.k = p.k; a.v = p.v; a.zk = p.zk; a.zv = p.zv;
  a.state_k = p.state_k; a.state_v = p.state_v;
  a.grid_k = p.grid_k; a.grid_v = p.grid_v;
  a.ring_k = p.ring_k; a.ring_v = p.ring_v;
  a.pos = p.pos; a.max_pos = p.max_pos; a.out = p.out;
  a.partials = p.partials; a.hdr = p.hdr;
  a.B = p.B; a.H = p.H; a.W = p.W;
  a.sl2 = p.scale * 1.4426950408889634f;
  a.reset_every = p.reset_every;
  a.heads = p.heads;
  if (p.bf16) {
    return p.Dh == 128 ? launch_typed<bf16_t, 128>(a, p.n_items, p.any_split, s)
                       : launch_typed<bf16_t, 64>(a, p.n_items, p.any_split, s);
  }
  return p.Dh == 128 ? launch_typed<float, 128>(a, p.n_items, p.any_split, s)
                     : launch_typed<float, 64>(a, p.n_items, p.any_split, s);
}

}  // namespace rat
