// Dilated prefill attention over recurrent states.
//
// Query t of a head with dilation D and local window W attends to the
// recurrent states at
//     S_t = { j <= t : (j + 1) mod D == 0 }  U  { max(0, t-W+1) .. t }
// ("RAT+: Train Dense, Infer Sparse", abstract and Fig. 1c: dilated attention
// over every D-th state, optionally with a local window; "Augmenting Attention
// with Exponentially Decaying Memory ...", section 2.2: attention runs over
// the memory states K~, V~).  An empty S_t yields a zero output row.
//
// The key set splits into two disjoint ranges:
//   grid   : grid entries i < n_g(t) = max(0, t - W + 1) / D  (entry i is the
//            state at position (i + 1) * D - 1; with W > 0 only entries
//            strictly older than the window, with W = 0 every grid entry <= t)
//   window : positions max(0, t - W + 1) .. t (W > 0 only).
// The pages' GH200 path uses FlexAttention with a dilated mask; this is a
// gfx950-native kernel: a q-tile walks the compact grid tiles (only the tile
// holding the n_g boundary is masked) and then the window band.
//
// bf16 kernel.  Block = 4 waves x 32 queries.  Per 64-key tile each wave
// computes S^T = K Q^T on v_mfma_f32_32x32x16_bf16 (keys on M, queries on N),
// so that after the online softmax its fp32 accumulators, converted to bf16,
// are already the B operand of O^T = V^T P^T: no shuffles between the two
// products.  K is staged row-major in LDS (rows padded to 272 B, conflict-free
// 16-byte fragment reads); V is transposed while staged (key pairs packed into
// dwords, XOR-swizzled columns) so that V^T fragments are two 8-byte LDS
// reads.  Softmax runs in base 2 with the scale folded into one FMA.  Block
// order is heaviest q-tile first and keeps each (b, h) pair on one XCD.
//
// fp32 kernel.  A plain exact-fp32 path (one or two lanes per query, keys
// staged in LDS) for fp32 inputs.
#include "rat_internal.h"

namespace rat {
namespace {

constexpr int kBM = 128;      // queries per block (bf16 kernel)
constexpr int kBN = 64;       // keys per tile
constexpr int kKRow = 136;    // LDS K row: 128 bf16 + 8 pad (272 B)

struct AttnArgs {
  const void* q;
  void* out;
  const void* grid_k;
  const void* grid_v;
  const void* all_k;
  const void* all_v;
  int B, T, H, W;
  int n_qtiles;
  float sl2;                  // softmax scale * log2(e)
  HeadTable heads;
};

__device__ __forceinline__ int n_grid(int t, int W, int D) {
  const int x = t - W + 1;
  return x > 0 ? x / D : 0;
}

// Block -> (b, h, q-tile): heaviest q-tile first; when B*H is a multiple of
// 8 every (b, h) pair stays on one XCD (blocks are dispatched round-robin
// over the 8 XCDs), so its K/V tiles are shared through that XCD's L2.
__device__ __forceinline__ void block_coords(int bid, int B, int H, int n_qtiles, int& b, int& h,
                                             int& qtile) {
  const int BH = B * H;
  int r, p;
  if (BH % 8 == 0) {
    const int xcd = bid & 7;
    const int k = bid >> 3;
    const int npx = BH >> 3;
    r = k / npx;
    p = xcd + 8 * (k - r * npx);
  } else {
    r = bid / BH;
    p = bid - r * BH;
  }
  qtile = n_qtiles - 1 - r;
  b = p / H;
  h = p - b * H;
}

__device__ __forceinline__ int vt_swz(int d) { return 2 * ((d ^ (d >> 3)) & 15); }

// ---------------------------------------------------------------------------
// bf16 MFMA kernel
// ---------------------------------------------------------------------------
template <int DH>
__global__ __launch_bounds__(256) void attn_bf16_kernel(const AttnArgs a) {
  constexpr int KS = DH / 16;            // MFMA k-steps over the head dim
  constexpr int DB = DH / 32;            // 32-wide d blocks of O^T
  constexpr int CH = DH / 8;             // 16-byte chunks per row
  constexpr int KT = (kBN * CH) / 256;   // K staging tasks per thread
  constexpr int VT = (kBN / 2 * CH) / 256;  // V staging tasks (key pairs) per thread
  static_assert(KT >= 1 && VT >= 1, "tile shape");

  __shared__ __attribute__((aligned(16))) bf16_t sK[kBN * kKRow];
  __shared__ __attribute__((aligned(16))) uint32_t sVt[DH * (kBN / 2)];

  int b, h, qtile;
  block_coords(blockIdx.x, a.B, a.H, a.n_qtiles, b, h, qtile);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int n = lane & 31;
  const int g = lane >> 5;
  const int T = a.T, H = a.H, W = a.W;
  const int D = a.heads.dil[h];
  const int64_t rowC = (int64_t)H * DH;   // elements between tokens

  const int t0 = qtile * kBM;
  const int t_last = min(t0 + kBM, T) - 1;
  const int tq = t0 + wave * 32 + n;      // this lane's query (column of S^T)
  const bool q_live = tq < T;

  // Q^T fragments (B operand): query tq, head dims 16*ks + 8*g .. +7
  bf16x8_t qf[KS];
  {
    const bf16_t* qp = static_cast<const bf16_t*>(a.q) + ((int64_t)b * T + tq) * rowC + h * DH;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      uint4 w = q_live ? *reinterpret_cast<const uint4*>(qp + 16 * ks + 8 * g) : make_uint4(0, 0, 0, 0);
      qf[ks] = __builtin_bit_cast(bf16x8_t, w);
    }
  }

  // key ranges of the block
  const int ng_hi = n_grid(t_last, W, D);
  const int ng_lo = n_grid(t0, W, D);
  const int ng_me = q_live ? n_grid(tq, W, D) : 0;
  const int ntile_g = (ng_hi + kBN - 1) / kBN;
  const int j_lo = W > 0 ? max(0, t0 - W + 1) : 0;
  const int ntile_w = W > 0 ? (t_last - j_lo + kBN) / kBN : 0;
  const int ntiles = ntile_g + ntile_w;
  const int win_lo_me = max(0, tq - W + 1);

  const bf16_t* gk = static_cast<const bf16_t*>(a.grid_k) + grid_row_offset(a.heads, a.B, b, h, 0, DH);
  const bf16_t* gv = static_cast<const bf16_t*>(a.grid_v) + grid_row_offset(a.heads, a.B, b, h, 0, DH);
  const bf16_t* ak = W > 0 ? static_cast<const bf16_t*>(a.all_k) + (int64_t)b * T * rowC + h * DH : nullptr;
  const bf16_t* av = W > 0 ? static_cast<const bf16_t*>(a.all_v) + (int64_t)b * T * rowC + h * DH : nullptr;

  uint4 kreg[KT];
  uint4 vreg[VT][2];

  auto prefetch = [&](int it) {
    const bf16_t* kb;
    const bf16_t* vb;
    int64_t stride;
    int row0, nvalid;
    if (it < ntile_g) {
      kb = gk; vb = gv; stride = DH; row0 = it * kBN; nvalid = ng_hi - row0;
    } else {
      kb = ak; vb = av; stride = rowC; row0 = j_lo + (it - ntile_g) * kBN; nvalid = t_last + 1 - row0;
    }
#pragma unroll
    for (int k = 0; k < KT; ++k) {
      const int task = tid + 256 * k;
      const int c = task % CH;
      const int r = task / CH;
      kreg[k] = r < nvalid ? *reinterpret_cast<const uint4*>(kb + (int64_t)(row0 + r) * stride + 8 * c)
                           : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int k = 0; k < VT; ++k) {
      const int task = tid + 256 * k;
      const int c = task % CH;
      const int kp = task / CH;
      const int r = 2 * kp;
      vreg[k][0] = r < nvalid ? *reinterpret_cast<const uint4*>(vb + (int64_t)(row0 + r) * stride + 8 * c)
                              : make_uint4(0, 0, 0, 0);
      vreg[k][1] = r + 1 < nvalid ? *reinterpret_cast<const uint4*>(vb + (int64_t)(row0 + r + 1) * stride + 8 * c)
                                  : make_uint4(0, 0, 0, 0);
    }
  };

  auto commit = [&]() {
#pragma unroll
    for (int k = 0; k < KT; ++k) {
      const int task = tid + 256 * k;
      const int c = task % CH;
      const int r = task / CH;
      *reinterpret_cast<uint4*>(sK + r * kKRow + 8 * c) = kreg[k];
    }
#pragma unroll
    for (int k = 0; k < VT; ++k) {
      const int task = tid + 256 * k;
      const int c = task % CH;
      const int kp = task / CH;
      const uint32_t w0[4] = {vreg[k][0].x, vreg[k][0].y, vreg[k][0].z, vreg[k][0].w};
      const uint32_t w1[4] = {vreg[k][1].x, vreg[k][1].y, vreg[k][1].z, vreg[k][1].w};
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int d = 8 * c + i;
        // low half: key 2kp, high half: key 2kp+1, head dim d
        const uint32_t packed = (i & 1) ? __builtin_amdgcn_perm(w1[i >> 1], w0[i >> 1], 0x07060302u)
                                        : __builtin_amdgcn_perm(w1[i >> 1], w0[i >> 1], 0x05040100u);
        sVt[d * (kBN / 2) + (kp ^ vt_swz(d))] = packed;
      }
    }
  };

  floatx16_t o[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[i][r] = 0.f;
  float m_run = -INFINITY;
  float l_run = 0.f;

  if (ntiles > 0) prefetch(0);
  for (int it = 0; it < ntiles; ++it) {
    __syncthreads();
    commit();
    __syncthreads();
    if (it + 1 < ntiles) prefetch(it + 1);

    // ---- S^T = K Q^T for two 32-key blocks
    floatx16_t s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) s[kb][r] = 0.f;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const uint4 w = *reinterpret_cast<const uint4*>(sK + (32 * kb + n) * kKRow + 16 * ks + 8 * g);
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, w), qf[ks], s[kb], 0, 0, 0);
      }
    }

    // ---- mask (boundary grid tile, every window tile)
    const bool is_grid = it < ntile_g;
    if (is_grid) {
      const int i0 = it * kBN;
      if (i0 + kBN > ng_lo) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int kk = 32 * kb + 8 * (r >> 2) + 4 * g + (r & 3);
            if (i0 + kk >= ng_me) s[kb][r] = -INFINITY;
          }
      }
    } else {
      const int j0 = j_lo + (it - ntile_g) * kBN;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int j = j0 + 32 * kb + 8 * (r >> 2) + 4 * g + (r & 3);
          if (j < win_lo_me || j > tq) s[kb][r] = -INFINITY;
        }
    }

    // ---- online softmax (base 2; running max shared by the two lane halves)
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx * a.sl2);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
    m_run = m_new;
    float psum = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = __builtin_amdgcn_exp2f(fmaf(s[kb][r], a.sl2, -m_use));
        s[kb][r] = p;
        psum += p;
      }
    l_run = l_run * alpha + psum;
#pragma unroll
    for (int i = 0; i < DB; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[i][r] *= alpha;

    // ---- O^T += V^T P^T over four 16-key steps
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      const int kb = st >> 1;
      const int r0 = 8 * (st & 1);
      uint4 pw;
      pw.x = pack_bf16x2(s[kb][r0 + 0], s[kb][r0 + 1]);
      pw.y = pack_bf16x2(s[kb][r0 + 2], s[kb][r0 + 3]);
      pw.z = pack_bf16x2(s[kb][r0 + 4], s[kb][r0 + 5]);
      pw.w = pack_bf16x2(s[kb][r0 + 6], s[kb][r0 + 7]);
      const bf16x8_t pf = __builtin_bit_cast(bf16x8_t, pw);
      const int kp0 = 8 * st + 2 * g;      // keys 16st + 4g .. +3
      const int kp1 = kp0 + 4;             // keys 16st + 8 + 4g .. +3
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const int d = 32 * db + n;
        const int sw = vt_swz(d);
        const uint2 lo = *reinterpret_cast<const uint2*>(sVt + d * (kBN / 2) + (kp0 ^ sw));
        const uint2 hi = *reinterpret_cast<const uint2*>(sVt + d * (kBN / 2) + (kp1 ^ sw));
        const uint4 vw = make_uint4(lo.x, lo.y, hi.x, hi.y);
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, vw), pf, o[db], 0, 0, 0);
      }
    }
  }

  // ---- normalise and store (empty key set -> zeros)
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
  if (q_live) {
    bf16_t* op = static_cast<bf16_t*>(a.out) + ((int64_t)b * T + tq) * rowC + h * DH;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int k4 = 0; k4 < 4; ++k4) {
        const int d = 32 * db + 8 * k4 + 4 * g;
        const uint2 w = make_uint2(pack_bf16x2(o[db][4 * k4 + 0] * inv, o[db][4 * k4 + 1] * inv),
                                   pack_bf16x2(o[db][4 * k4 + 2] * inv, o[db][4 * k4 + 3] * inv));
        *reinterpret_cast<uint2*>(op + d) = w;
      }
  }
}

// ---------------------------------------------------------------------------
// fp32 kernel: exact fp32 arithmetic, TPQ = DH / 64 lanes per query
// ---------------------------------------------------------------------------
constexpr int kF32Keys = 32;

template <int DH>
__global__ __launch_bounds__(64 * (DH / 64)) void attn_f32_kernel(const AttnArgs a) {
  constexpr int TPQ = DH / 64;
  constexpr int NT = 64 * TPQ;
  __shared__ __attribute__((aligned(16))) float sK[kF32Keys][DH];
  __shared__ __attribute__((aligned(16))) float sV[kF32Keys][DH];

  int b, h, qtile;
  block_coords(blockIdx.x, a.B, a.H, a.n_qtiles, b, h, qtile);
  const int tid = threadIdx.x;
  const int qi = tid / TPQ;
  const int part = tid - qi * TPQ;      // which 64 head dims
  const int T = a.T, H = a.H, W = a.W;
  const int D = a.heads.dil[h];
  const int64_t rowC = (int64_t)H * DH;
  const int t0 = qtile * 64;
  const int t_last = min(t0 + 64, T) - 1;
  const int tq = t0 + qi;
  const bool q_live = tq < T;

  float q[64], acc[64];
  {
    const float* qp = static_cast<const float*>(a.q) + ((int64_t)b * T + tq) * rowC + h * DH + 64 * part;
#pragma unroll
    for (int i = 0; i < 64; i += 4) {
      float4 w = q_live ? *reinterpret_cast<const float4*>(qp + i) : make_float4(0.f, 0.f, 0.f, 0.f);
      q[i] = w.x; q[i + 1] = w.y; q[i + 2] = w.z; q[i + 3] = w.w;
    }
#pragma unroll
    for (int i = 0; i < 64; ++i) acc[i] = 0.f;
  }
  const int ng_hi = n_grid(t_last, W, D);
  const int ng_me = q_live ? n_grid(tq, W, D) : 0;
  const int ntile_g = (ng_hi + kF32Keys - 1) / kF32Keys;
  const int j_lo = W > 0 ? max(0, t0 - W + 1) : 0;
  const int ntile_w = W > 0 ? (t_last - j_lo + kF32Keys) / kF32Keys : 0;
  const int win_lo_me = max(0, tq - W + 1);
  const float* gk = static_cast<const float*>(a.grid_k) + grid_row_offset(a.heads, a.B, b, h, 0, DH);
  const float* gv = static_cast<const float*>(a.grid_v) + grid_row_offset(a.heads, a.B, b, h, 0, DH);
  const float* ak = W > 0 ? static_cast<const float*>(a.all_k) + (int64_t)b * T * rowC + h * DH : nullptr;
  const float* av = W > 0 ? static_cast<const float*>(a.all_v) + (int64_t)b * T * rowC + h * DH : nullptr;

  float m_run = -INFINITY, l_run = 0.f;
  for (int it = 0; it < ntile_g + ntile_w; ++it) {
    const float* kb;
    const float* vb;
    int64_t stride;
    int row0, nvalid;
    const bool is_grid = it < ntile_g;
    if (is_grid) {
      kb = gk; vb = gv; stride = DH; row0 = it * kF32Keys; nvalid = ng_hi - row0;
    } else {
      kb = ak; vb = av; stride = rowC; row0 = j_lo + (it - ntile_g) * kF32Keys; nvalid = t_last + 1 - row0;
    }
    __syncthreads();
    for (int e = tid * 4; e < kF32Keys * DH; e += NT * 4) {
      const int r = e / DH;
      const int c = e - r * DH;
      float4 kw = make_float4(0.f, 0.f, 0.f, 0.f), vw = kw;
      if (r < nvalid) {
        kw = *reinterpret_cast<const float4*>(kb + (int64_t)(row0 + r) * stride + c);
        vw = *reinterpret_cast<const float4*>(vb + (int64_t)(row0 + r) * stride + c);
      }
      *reinterpret_cast<float4*>(&sK[r][c]) = kw;
      *reinterpret_cast<float4*>(&sV[r][c]) = vw;
    }
    __syncthreads();
    for (int kk = 0; kk < kF32Keys; ++kk) {
      bool valid;
      if (is_grid) {
        valid = row0 + kk < ng_me;
      } else {
        const int j = row0 + kk;
        valid = j >= win_lo_me && j <= tq && kk < nvalid;
      }
      float sp = 0.f;
#pragma unroll
      for (int i = 0; i < 64; ++i) sp = fmaf(q[i], sK[kk][64 * part + i], sp);
      if (TPQ == 2) sp += __shfl_xor(sp, 1);
      if (valid) {   // uniform across the lanes of one query
        const float sc = sp * a.sl2;
        const float m_new = fmaxf(m_run, sc);
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
        const float p = __builtin_amdgcn_exp2f(sc - m_new);
        l_run = l_run * alpha + p;
#pragma unroll
        for (int i = 0; i < 64; ++i) acc[i] = fmaf(p, sV[kk][64 * part + i], acc[i] * alpha);
        m_run = m_new;
      }
    }
  }
  if (q_live) {
    const float inv = l_run > 0.f ? 1.0f / l_run : 0.f;
    float* op = static_cast<float*>(a.out) + ((int64_t)b * T + tq) * rowC + h * DH + 64 * part;
#pragma unroll
    for (int i = 0; i < 64; i += 4)
      *reinterpret_cast<float4*>(op + i) = make_float4(acc[i] * inv, acc[i + 1] * inv, acc[i + 2] * inv, acc[i + 3] * inv);
  }
}

int xcd_padded_blocks(int BH, int n_qtiles) {
  if (BH % 8 == 0) return BH * n_qtiles;   // exact: npx = BH / 8 pairs per XCD
  return BH * n_qtiles;
}

}  // namespace

hipError_t launch_prefill_attention(const AttnPlan& p, hipStream_t s) {
  if (p.T <= 0 || p.B <= 0) return hipSuccess;
  AttnArgs a;
  a.q = p.q; a.out = p.out;
  a.grid_k = p.grid_k; a.grid_v = p.grid_v;
  a.all_k = p.all_k; a.all_v = p.all_v;
  a.B = p.B; a.T = p.T; a.H = p.H; a.W = p.W;
  a.sl2 = p.scale * 1.4426950408889634f;
  a.heads = p.heads;
  const int BH = p.B * p.H;
  if (p.bf16) {
    a.n_qtiles = (p.T + kBM - 1) / kBM;
    const int blocks = xcd_padded_blocks(BH, a.n_qtiles);
    if (p.Dh == 128)
      hipLaunchKernelGGL(attn_bf16_kernel<128>, dim3(blocks), dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL(attn_bf16_kernel<64>, dim3(blocks), dim3(256), 0, s, a);
  } else {
    a.n_qtiles = (p.T + 63) / 64;
    const int blocks = xcd_padded_blocks(BH, a.n_qtiles);
    if (p.Dh == 128)
      hipLaunchKernelGGL(attn_f32_kernel<128>, dim3(blocks), dim3(128), 0, s, a);
    else
      hipLaunchKernelGGL(attn_f32_kernel<64>, dim3(blocks), dim3(64), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace rat
