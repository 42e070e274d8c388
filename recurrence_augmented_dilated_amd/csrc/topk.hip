// Top-k block attention over RAT+ memory states.
//
// "Augmenting Attention with Exponentially Decaying Memory Improves
// Query-Aware KV Sparsity", section 2.2: query-aware sparse inference scores
// KV blocks, keeps the best ones and attends only over them; with RAT+ it runs
// on the memory states (K~, V~).  Block representatives (section 3, sparse
// inference settings; "RAT+: Train Dense, Infer Sparse", Fig. 3 and Tables
// 17-18): Quest keeps the dimension-wise min and max of a block's key states
// and scores sum_d max(q_d min_d, q_d max_d); MoBA keeps their mean and
// scores q . mean.  The first block and the query's own block are always
// attended; the top-k complete blocks between them are added (ties to the
// lower block index).
//
// Every recurrent state sits in a cache [H][B][max_pos][Dh]; the summaries
// of complete blocks in fp32 [H][B][max_pos / block][3][Dh].  The general
// path gives one workgroup to one query: it scores the candidate blocks from
// the summaries into LDS, takes the top k by rank (up to 1024 candidates) or
// by repeated wave-wide argmax, then streams the rows of the kept blocks
// (Dh / 8 lanes per row, online softmax per lane group, waves merged in LDS).
// Prefill with 64-position blocks from position 0 only selects here, a tile
// of 64 queries per workgroup (they share their candidates), and attends on
// the MFMA prefill attention kernel with the chosen lists.
#include "rat_internal.h"
#include "kv_stream.h"

namespace rat {
namespace {

constexpr int kAW = 4;        // waves per attend workgroup
constexpr int kAUnroll = 8;   // row steps in flight per wave

template <typename ET> __device__ __forceinline__ float ld1(const ET* p);
template <> __device__ __forceinline__ float ld1<bf16_t>(const bf16_t* p) { return bf16_to_f32(*p); }
template <> __device__ __forceinline__ float ld1<float>(const float* p) { return *p; }
template <typename ET> __device__ __forceinline__ void st1(ET* p, float x);
template <> __device__ __forceinline__ void st1<bf16_t>(bf16_t* p, float x) { *p = bf16_t(pack_bf16x2(x, 0.f) & 0xffffu); }
template <> __device__ __forceinline__ void st1<float>(float* p, float x) { *p = x; }

__device__ __forceinline__ int64_t cache_off(int B, int64_t max_pos, int h, int b, int64_t row, int Dh) {
  return (((int64_t)h * B + b) * max_pos + row) * Dh;
}
__device__ __forceinline__ int64_t summary_off(int B, int64_t nbcap, int h, int b, int64_t j, int Dh) {
  return (((int64_t)h * B + b) * nbcap + j) * 3 * Dh;
}

// ---- summaries of complete blocks: one workgroup of 256 threads per
// (h, b, j); a thread takes two adjacent dims of every G-th row of the block
// (G = 512 / Dh row groups), the groups are combined in LDS in group order
constexpr int kStatsThreads = 256;

template <typename ET>
__global__ __launch_bounds__(kStatsThreads) void topk_stats_kernel(const TopkPlan p, int64_t j_lo, int64_t nj) {
  __shared__ float s_red[3][2 * kStatsThreads];   // [min, max, sum][group * Dh + dim]
  const int64_t id = blockIdx.x;
  const int64_t jj = id % nj;
  const int64_t hb = id / nj;
  const int b = int(hb % p.B);
  const int h = int(hb / p.B);
  const int64_t j = j_lo + jj;
  const int tid = threadIdx.x;
  const int half = p.Dh / 2;
  const int G = 2 * kStatsThreads / p.Dh;
  const int rg = tid / half;
  const int d = 2 * (tid - rg * half);
  const ET* src = static_cast<const ET*>(p.cache_k) + cache_off(p.B, p.max_pos, h, b, j * p.block, p.Dh) + d;
  float mn0 = INFINITY, mx0 = -INFINITY, sm0 = 0.f, mn1 = INFINITY, mx1 = -INFINITY, sm1 = 0.f;
#pragma unroll 4
  for (int r = rg; r < p.block; r += G) {
    float x0, x1;
    if constexpr (sizeof(ET) == 2) {
      const uint32_t w = *reinterpret_cast<const uint32_t*>(src + (int64_t)r * p.Dh);
      x0 = bf16_lo(w);
      x1 = bf16_hi(w);
    } else {
      const float2 w = *reinterpret_cast<const float2*>(src + (int64_t)r * p.Dh);
      x0 = w.x;
      x1 = w.y;
    }
    mn0 = fminf(mn0, x0); mx0 = fmaxf(mx0, x0); sm0 += x0;
    mn1 = fminf(mn1, x1); mx1 = fmaxf(mx1, x1); sm1 += x1;
  }
  const int o = rg * p.Dh + d;
  s_red[0][o] = mn0; s_red[0][o + 1] = mn1;
  s_red[1][o] = mx0; s_red[1][o + 1] = mx1;
  s_red[2][o] = sm0; s_red[2][o + 1] = sm1;
  __syncthreads();
  if (tid < p.Dh) {
    float mn = INFINITY, mx = -INFINITY, sum = 0.f;
    for (int g = 0; g < G; ++g) {
      mn = fminf(mn, s_red[0][g * p.Dh + tid]);
      mx = fmaxf(mx, s_red[1][g * p.Dh + tid]);
      sum += s_red[2][g * p.Dh + tid];
    }
    float* dst = p.summary + summary_off(p.B, p.max_pos / p.block, h, b, j, p.Dh) + tid;
    dst[0] = mn;
    dst[p.Dh] = mx;
    dst[2 * p.Dh] = sum / float(p.block);
  }
}

// ---- decode: state update, cache row, summary of a block the row completes
template <typename ET>
__global__ void topk_append_kernel(const TopkAppendPlan p) {
  const int bh = blockIdx.x;
  const int b = bh / p.H;
  const int h = bh - b * p.H;
  const int d = threadIdx.x;
  const int64_t t = p.pos[b];
  if (t < 0 || t >= p.max_pos) {
    if (d == 0) atomicOr(&p.hdr[2], kErrDecodePos);
    return;
  }
  const int64_t idx = (int64_t)bh * p.Dh + d;
  float gk, ck, gv, cv;
  gate_pair(p.zk[idx], gk, ck);
  gate_pair(p.zv[idx], gv, cv);
  const float sk = gk * p.state_k[idx] + ck * ld1<ET>(static_cast<const ET*>(p.k) + idx);
  const float sv = gv * p.state_v[idx] + cv * ld1<ET>(static_cast<const ET*>(p.v) + idx);
  p.state_k[idx] = sk;
  p.state_v[idx] = sv;
  ET* ck_row = static_cast<ET*>(p.cache_k) + cache_off(p.B, p.max_pos, h, b, t, p.Dh) + d;
  st1<ET>(ck_row, sk);
  st1<ET>(static_cast<ET*>(p.cache_v) + cache_off(p.B, p.max_pos, h, b, t, p.Dh) + d, sv);
  if ((t + 1) % p.block == 0) {
    // block j = (t+1)/block - 1 is complete: rows before t from the cache,
    // row t as just stored (rounded to the cache type)
    const int64_t j = (t + 1) / p.block - 1;
    const ET* src = static_cast<const ET*>(p.cache_k) + cache_off(p.B, p.max_pos, h, b, j * p.block, p.Dh) + d;
    float mn = INFINITY, mx = -INFINITY, sum = 0.f;
    for (int r = 0; r < p.block; ++r) {
      float x;
      if (r == p.block - 1) {
        ET tmp;
        st1<ET>(&tmp, sk);
        x = ld1<ET>(&tmp);
      } else {
        x = ld1<ET>(src + (int64_t)r * p.Dh);
      }
      mn = fminf(mn, x);
      mx = fmaxf(mx, x);
      sum += x;
    }
    float* dst = p.summary + summary_off(p.B, p.max_pos / p.block, h, b, j, p.Dh) + d;
    dst[0] = mn;
    dst[p.Dh] = mx;
    dst[2 * p.Dh] = sum / float(p.block);
  }
}

// better(v, j) than (bv, bi): higher score, ties to the lower index; NaN marks
// a candidate already taken
__device__ __forceinline__ bool better(float v, int j, float bv, int bi) {
  return v == v && (v > bv || (v == bv && j < bi));
}

// ---- selection for a tile of 64 queries (block size 64, positions from 0):
// the tile's queries share one block and hence one candidate set, so the
// candidates' summaries are read once per tile.  A lane holds one query
// (its row in registers); each wave scores every fourth candidate of a
// 32-candidate chunk staged in LDS (broadcast reads), in fp32 like the
// per-query kernel; then a wave per query ranks the candidates (higher
// score, ties to the lower index) and writes the kept ones in ascending
// order with a ballot prefix.
constexpr int kTileQ = 64;
constexpr int kTileChunk = 32;

// unsigned key with the order of the float scores (no NaN here); -0 and +0,
// equal as scores, share one key
__device__ __forceinline__ uint32_t order_key(float f) {
  const uint32_t u = __float_as_uint(f + 0.f);   // -0 + 0 = +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

template <int DH>
__global__ __launch_bounds__(kAW * 64) void topk_select_tile_kernel(const TopkPlan p, int ncap) {
  extern __shared__ float s_tsc[];   // [kTileQ][ncap] candidate scores
  __shared__ __attribute__((aligned(16))) float s_st[2][kTileChunk][DH];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int ntile = (p.T + kTileQ - 1) / kTileQ;
  const int BH = p.B * p.H;
  const int tile = ntile - 1 - int(blockIdx.x / BH);   // heaviest tiles first
  const int bh = int(blockIdx.x % BH);
  const int b = bh / p.H;
  const int h = bh - b * p.H;
  const int ncand = tile > 1 ? tile - 1 : 0;           // candidate blocks 1 .. tile-1
  const int t = tile * kTileQ + lane;
  const bool live = t < p.T;

  // this lane's query (fp32)
  float qv[DH];
  {
    const bf16_t* qp = static_cast<const bf16_t*>(p.q) + (((int64_t)b * p.T + (live ? t : 0)) * p.H + h) * DH;
#pragma unroll
    for (int i = 0; i < DH / 8; ++i) {
      const uint4 w = *reinterpret_cast<const uint4*>(qp + 8 * i);
      const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        qv[8 * i + 2 * k] = bf16_lo(u[k]);
        qv[8 * i + 2 * k + 1] = bf16_hi(u[k]);
      }
    }
  }

  const int64_t nbcap = p.max_pos / p.block;
  const float* sb = p.summary + summary_off(p.B, nbcap, h, b, 0, DH);
  const bool quest = p.score == kTopkQuest;
  for (int c0 = 0; c0 < ncand; c0 += kTileChunk) {
    const int nc = min(kTileChunk, ncand - c0);
    // stage the chunk: Quest min and max, MoBA mean
    for (int e = tid; e < nc * (DH / 4); e += kAW * 64) {
      const int ci = e / (DH / 4), d4 = e - ci * (DH / 4);
      const float* src = sb + (int64_t)(c0 + 1 + ci) * 3 * DH + 4 * d4;
      if (quest) {
        *reinterpret_cast<float4*>(&s_st[0][ci][4 * d4]) = *reinterpret_cast<const float4*>(src);
        *reinterpret_cast<float4*>(&s_st[1][ci][4 * d4]) = *reinterpret_cast<const float4*>(src + DH);
      } else {
        *reinterpret_cast<float4*>(&s_st[0][ci][4 * d4]) = *reinterpret_cast<const float4*>(src + 2 * DH);
      }
    }
    __syncthreads();
    for (int ci = wave; ci < nc; ci += kAW) {
      float sc = 0.f;
      if (quest) {
#pragma unroll
        for (int d4 = 0; d4 < DH / 4; ++d4) {
          const float4 mn = *reinterpret_cast<const float4*>(&s_st[0][ci][4 * d4]);
          const float4 mx = *reinterpret_cast<const float4*>(&s_st[1][ci][4 * d4]);
          sc += fmaxf(qv[4 * d4] * mn.x, qv[4 * d4] * mx.x);
          sc += fmaxf(qv[4 * d4 + 1] * mn.y, qv[4 * d4 + 1] * mx.y);
          sc += fmaxf(qv[4 * d4 + 2] * mn.z, qv[4 * d4 + 2] * mx.z);
          sc += fmaxf(qv[4 * d4 + 3] * mn.w, qv[4 * d4 + 3] * mx.w);
        }
      } else {
#pragma unroll
        for (int d4 = 0; d4 < DH / 4; ++d4) {
          const float4 me = *reinterpret_cast<const float4*>(&s_st[0][ci][4 * d4]);
          sc = fmaf(qv[4 * d4], me.x, sc);
          sc = fmaf(qv[4 * d4 + 1], me.y, sc);
          sc = fmaf(qv[4 * d4 + 2], me.z, sc);
          sc = fmaf(qv[4 * d4 + 3], me.w, sc);
        }
      }
      s_tsc[lane * ncap + c0 + ci] = sc == sc ? sc : -INFINITY;
    }
    __syncthreads();
  }

  // a wave per query: ranks, then the kept blocks in ascending order
  const int nsel = ncand < p.topk ? ncand : p.topk;
  for (int qi = wave; qi < kTileQ; qi += kAW) {
    const int tq = tile * kTileQ + qi;
    if (tq >= p.T) break;
    int32_t* cp = p.chosen + (((int64_t)b * p.T + tq) * p.H + h) * p.topk;
    const float* row = s_tsc + qi * ncap;
    int base = 0;
    if (ncand <= p.topk) {
      for (int j = lane; j < ncand; j += 64) cp[j] = j + 1;
      base = ncand;
    } else if (ncand <= 64) {
      // one candidate per lane: the nsel-th highest score is found bit by bit
      // on an order-preserving integer key (wave-wide ballot counts); kept
      // are the candidates above it, then the lowest indices equal to it
      const uint32_t key = lane < ncand ? order_key(row[lane]) : 0u;   // 0: below every real key
      uint32_t thr = 0;
#pragma unroll
      for (int bit = 31; bit >= 0; --bit) {
        const uint32_t cand = thr | (1u << bit);
        if (__builtin_popcountll(__ballot(key >= cand)) >= nsel) thr = cand;
      }
      const uint64_t gt = __ballot(key > thr);
      uint64_t eq = __ballot(key == thr), take = 0;
      for (int ties = nsel - __builtin_popcountll(gt); ties > 0; --ties) {
        const uint64_t low = eq & (~eq + 1ull);
        take |= low;
        eq ^= low;
      }
      const uint64_t m = gt | take;   // nsel bits
      if ((m >> lane) & 1ull) cp[__builtin_popcountll(m & ((1ull << lane) - 1ull))] = lane + 1;
      base = nsel;
    } else {
      for (int j0 = 0; j0 < ncand; j0 += 64) {
        const int j = j0 + lane;
        const bool in = j < ncand;
        const float v = in ? row[j] : 0.f;
        int r = 0;
        // the other candidates 64 at a time: one LDS read per lane, then each
        // entry broadcast from its lane by a scalar read (no LDS round trip
        // per comparison)
        for (int i0 = 0; i0 < ncand; i0 += 64) {
          const int ucnt = min(64, ncand - i0);
          const int uc = __float_as_int(lane < ucnt ? row[i0 + lane] : 0.f);
#pragma unroll 8
          for (int ii = 0; ii < ucnt; ++ii) {
            const float u = __int_as_float(__builtin_amdgcn_readlane(uc, ii));
            const int i = i0 + ii;
            r += (u > v || (u == v && i < j)) ? 1 : 0;
          }
        }
        const bool kept = in && r < nsel;
        const uint64_t m = __ballot(kept);
        if (kept) cp[base + __builtin_popcountll(m & ((1ull << lane) - 1ull))] = j + 1;
        base += __builtin_popcountll(m);
      }
    }
    for (int j = base + lane; j < p.topk; j += 64) cp[j] = -1;
  }
}

// Candidate counts up to this may be selected by rank in one pass (when that
// costs less than the argmax rounds); otherwise by repeated wave-wide argmax.
constexpr int kRankMax = 1024;

// ---- selection and attention: one workgroup per query
// STREAM (decode): every kept row is read by this one query only, so the rows
// are read non-temporally; prefill queries share kept blocks through the cache.
template <typename ET, int DH, bool STREAM>
__global__ __launch_bounds__(kAW * 64) void topk_attend_kernel(const TopkPlan p) {
  using R = Row8<ET>;
  constexpr int LPK = DH / 8;      // lanes per row
  constexpr int KPW = 64 / LPK;    // rows per wave step
  __shared__ float s_q[DH];
  extern __shared__ float s_sc[];     // candidate scores: max_pos / block floats (launch-time size)
  __shared__ int s_list[kTopkMaxK + 2];
  __shared__ int16_t s_rank[kRankMax];
  __shared__ float s_m[kAW], s_l[kAW];
  __shared__ float s_acc[kAW][DH];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int rg = lane / LPK;
  const int c = lane - rg * LPK;

  // ---- the query
  int b, h;
  int64_t t, qrow;
  if (p.pos) {                       // decode: one token per sequence
    qrow = blockIdx.x;               // b * H + h
    b = int(qrow / p.H);
    h = int(qrow - (int64_t)b * p.H);
    t = p.pos[b];
  } else {                           // prefill: row (b * T + i) * H + h is position p0 + i
    qrow = blockIdx.x;
    h = int(qrow % p.H);
    const int64_t bi = qrow / p.H;
    b = int(bi / p.T);
    t = p.p0 + (bi - (int64_t)b * p.T);
  }
  const ET* qp = static_cast<const ET*>(p.q) + qrow * DH;
  ET* op = static_cast<ET*>(p.out) + qrow * DH;
  int32_t* cp = p.chosen ? p.chosen + qrow * p.topk : nullptr;
  if (t < 0 || t >= p.max_pos) {     // decode position out of range: zero row (error bit set by append)
    if (tid < DH) st1<ET>(op + tid, 0.f);
    if (cp && tid < p.topk) cp[tid] = -1;
    return;
  }
  if (tid < DH) s_q[tid] = ld1<ET>(qp + tid);
  __syncthreads();

  const int64_t local = t / p.block;
  const int ncand = int(local > 1 ? local - 1 : 0);   // candidate blocks 1 .. local-1
  const int64_t nbcap = p.max_pos / p.block;
  const float* sb = p.summary + summary_off(p.B, nbcap, h, b, 0, DH);

  // ---- scores of the candidates (score of block j + 1 in s_sc[j]): LPK
  // lanes per candidate, eight head dims per lane, 16-byte loads
  {
    float qd[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) qd[i] = s_q[8 * c + i];
    const int slot = wave * KPW + rg;                 // candidate slot of this lane group
    for (int j0 = 0; j0 < ncand; j0 += kAW * KPW) {
      const int j = j0 + slot;
      const bool ok = j < ncand;
      const float* st = sb + (int64_t)(ok ? j + 1 : 0) * 3 * DH + 8 * c;
      float part = 0.f;
      if (p.score == kTopkQuest) {
        const float4 a0 = reinterpret_cast<const float4*>(st)[0], a1 = reinterpret_cast<const float4*>(st)[1];
        const float4 b0 = reinterpret_cast<const float4*>(st + DH)[0], b1 = reinterpret_cast<const float4*>(st + DH)[1];
        const float mn[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
        const float mx[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
#pragma unroll
        for (int i = 0; i < 8; ++i) part += fmaxf(qd[i] * mn[i], qd[i] * mx[i]);
      } else {
        const float4 a0 = reinterpret_cast<const float4*>(st + 2 * DH)[0];
        const float4 a1 = reinterpret_cast<const float4*>(st + 2 * DH)[1];
        const float me[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
#pragma unroll
        for (int i = 0; i < 8; ++i) part = fmaf(qd[i], me[i], part);
      }
      const float sc = group_sum<LPK>(part);
      if (ok && c == 0) s_sc[j] = sc == sc ? sc : -INFINITY;   // NaN marks "taken" below
    }
  }
  __syncthreads();

  // ---- the top k (or all candidates when there are at most k), taken by
  // one wave: per round a wave-wide argmax, no workgroup barrier
  const int nsel = ncand < p.topk ? ncand : p.topk;
  if (ncand <= p.topk) {
    for (int j = tid; j < ncand; j += kAW * 64) s_list[1 + j] = j + 1;
  } else if (ncand <= kRankMax &&
             ncand * ((ncand + kAW * 64 - 1) / (kAW * 64)) < nsel * (ncand / 64 + 12)) {
    // rank of every candidate (cheaper than nsel argmax rounds for few
    // candidates): the number that beat it (higher score, ties to the lower
    // index); the kept ones are the ranks below nsel
    for (int j = tid; j < ncand; j += kAW * 64) {
      const float v = s_sc[j];
      int r = 0;
      for (int i = 0; i < ncand; ++i) {
        const float u = s_sc[i];
        r += (u > v || (u == v && i < j)) ? 1 : 0;
      }
      s_rank[j] = (int16_t)r;
    }
    __syncthreads();
    // in ascending block order: a kept candidate's slot counts the kept
    // candidates below it
    for (int j = tid; j < ncand; j += kAW * 64) {
      if (s_rank[j] < nsel) {
        int pos = 0;
        for (int i = 0; i < j; ++i) pos += s_rank[i] < nsel ? 1 : 0;
        s_list[1 + pos] = j + 1;
      }
    }
  } else if (wave == 0) {
    for (int r = 0; r < nsel; ++r) {
      float bv = -INFINITY;
      int bi = 0x7fffffff;
      for (int j = lane; j < ncand; j += 64) {
        const float v = s_sc[j];
        if (better(v, j, bv, bi)) { bv = v; bi = j; }
      }
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) {
        const float ov = __shfl_xor(bv, off);
        const int oi = __shfl_xor(bi, off);
        if (better(ov, oi, bv, bi)) { bv = ov; bi = oi; }
      }
      // every lane holds the winner; one lane marks it taken (the wave's
      // later LDS reads are ordered after this write)
      if (lane == 0) {
        s_list[1 + r] = bi + 1;
        s_sc[bi] = __builtin_nanf("");
      }
    }
    if (lane == 0) {   // ascending block order
      for (int i = 2; i <= nsel; ++i) {
        const int x = s_list[i];
        int k = i - 1;
        while (k >= 1 && s_list[k] > x) { s_list[k + 1] = s_list[k]; --k; }
        s_list[k + 1] = x;
      }
    }
  }
  __syncthreads();
  if (cp && tid < p.topk) cp[tid] = tid < nsel ? s_list[1 + tid] : -1;
  if (p.select_only) return;

  // ---- key blocks: first, chosen, local (block 0 alone when local == 0)
  const int nlist = local > 0 ? nsel + 2 : 1;
  auto list_block = [&](int e) -> int64_t {
    if (local == 0) return 0;
    if (e == 0) return 0;
    if (e == nlist - 1) return local;
    return s_list[e];
  };

  float q8[8];
  const float sl2 = p.scale * 1.4426950408889634f;
#pragma unroll
  for (int i = 0; i < 8; ++i) q8[i] = s_q[8 * c + i] * sl2;
  Soft sm;
  sm.m = -INFINITY;
  sm.l = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) sm.acc[i] = 0.f;

  const ET* kc = static_cast<const ET*>(p.cache_k) + cache_off(p.B, p.max_pos, h, b, 0, DH) + 8 * c;
  const ET* vc = static_cast<const ET*>(p.cache_v) + cache_off(p.B, p.max_pos, h, b, 0, DH) + 8 * c;
  for (int e = wave; e < nlist; e += kAW) {
    const int64_t blk = list_block(e);
    const int64_t r_lo = blk * p.block;
    const int64_t r_hi = min(r_lo + p.block, t + 1);   // the local block stops at t
    for (int64_t base = r_lo; base < r_hi; base += KPW * kAUnroll) {
      typename R::raw kr[kAUnroll], vr[kAUnroll];
#pragma unroll
      for (int u = 0; u < kAUnroll; ++u) {
        const int64_t r = base + u * KPW + rg;
        const bool ok = r < r_hi;
        kr[u] = ok ? (STREAM ? R::load_nt(kc + r * DH) : R::load(kc + r * DH)) : R::zero();
        vr[u] = ok ? (STREAM ? R::load_nt(vc + r * DH) : R::load(vc + r * DH)) : R::zero();
      }
      float sc[kAUnroll];
      float vv[kAUnroll][8];
#pragma unroll
      for (int u = 0; u < kAUnroll; ++u) {
        float kf[8];
        R::get(kr[u], kf);
        R::get(vr[u], vv[u]);
        float d0 = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) d0 = fmaf(q8[i], kf[i], d0);
        d0 = group_sum<LPK>(d0);
        sc[u] = (base + u * KPW + rg) < r_hi ? d0 : -INFINITY;
      }
      soft_update<kAUnroll>(sm, sc, vv);
    }
  }

  // ---- merge the lane groups of a wave, then the waves
#pragma unroll
  for (int off = LPK; off < 64; off <<= 1) {
    const float m2 = __shfl_xor(sm.m, off);
    const float l2 = __shfl_xor(sm.l, off);
    float a2[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) a2[i] = __shfl_xor(sm.acc[i], off);
    soft_merge(sm, m2, l2, a2);
  }
  if (rg == 0) {
    if (c == 0) { s_m[wave] = sm.m; s_l[wave] = sm.l; }
#pragma unroll
    for (int i = 0; i < 8; ++i) s_acc[wave][8 * c + i] = sm.acc[i];
  }
  __syncthreads();
  if (wave == 0 && rg == 0) {
    Soft fin;
    fin.m = s_m[0];
    fin.l = s_l[0];
#pragma unroll
    for (int i = 0; i < 8; ++i) fin.acc[i] = s_acc[0][8 * c + i];
#pragma unroll
    for (int w = 1; w < kAW; ++w) soft_merge(fin, s_m[w], s_l[w], &s_acc[w][8 * c]);
    const float inv = fin.l > 0.f ? 1.0f / fin.l : 0.f;
    float o8[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) o8[i] = fin.acc[i] * inv;
    R::store(op + 8 * c, o8);
  }
}

}  // namespace

hipError_t launch_topk_stats(const TopkPlan& p, int64_t j_lo, int64_t j_hi, hipStream_t s) {
  const int64_t nj = j_hi - j_lo;
  if (nj <= 0) return hipSuccess;
  const int64_t blocks = (int64_t)p.H * p.B * nj;
  if (p.bf16)
    hipLaunchKernelGGL(topk_stats_kernel<bf16_t>, dim3((unsigned)blocks), dim3(kStatsThreads), 0, s, p, j_lo, nj);
  else
    hipLaunchKernelGGL(topk_stats_kernel<float>, dim3((unsigned)blocks), dim3(kStatsThreads), 0, s, p, j_lo, nj);
  return hipGetLastError();
}

hipError_t launch_topk_append(const TopkAppendPlan& p, hipStream_t s) {
  const int blocks = p.B * p.H;
  if (p.bf16)
    hipLaunchKernelGGL(topk_append_kernel<bf16_t>, dim3(blocks), dim3(p.Dh), 0, s, p);
  else
    hipLaunchKernelGGL(topk_append_kernel<float>, dim3(blocks), dim3(p.Dh), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_topk_select_tile(const TopkPlan& p, hipStream_t s) {
  const int ntile = (p.T + kTileQ - 1) / kTileQ;
  const int ncap = (ntile > 2 ? ntile - 2 : 0) | 1;   // candidate slots per query row (odd: no bank conflicts)
  const size_t lds = sizeof(float) * (size_t)kTileQ * ncap;
  const dim3 grid((unsigned)(ntile * p.B * p.H)), threads(kAW * 64);
  if (p.Dh == 128) hipLaunchKernelGGL((topk_select_tile_kernel<128>), grid, threads, lds, s, p, ncap);
  else hipLaunchKernelGGL((topk_select_tile_kernel<64>), grid, threads, lds, s, p, ncap);
  return hipGetLastError();
}

hipError_t launch_topk_attend(const TopkPlan& p, hipStream_t s) {
  const int64_t blocks = p.pos ? (int64_t)p.B * p.H : (int64_t)p.B * p.T * p.H;
  if (blocks <= 0) return hipSuccess;
  const dim3 grid((unsigned)blocks), threads(kAW * 64);
  // candidate scores in dynamic LDS: at most max_pos / block of them
  const size_t lds = sizeof(float) * (size_t)(p.max_pos / p.block > 0 ? p.max_pos / p.block : 1);
  const bool dec = p.pos != nullptr;
  if (p.bf16) {
    if (p.Dh == 128) {
      if (dec) hipLaunchKernelGGL((topk_attend_kernel<bf16_t, 128, true>), grid, threads, lds, s, p);
      else hipLaunchKernelGGL((topk_attend_kernel<bf16_t, 128, false>), grid, threads, lds, s, p);
    } else {
      if (dec) hipLaunchKernelGGL((topk_attend_kernel<bf16_t, 64, true>), grid, threads, lds, s, p);
      else hipLaunchKernelGGL((topk_attend_kernel<bf16_t, 64, false>), grid, threads, lds, s, p);
    }
  } else {
    if (p.Dh == 128) {
      if (dec) hipLaunchKernelGGL((topk_attend_kernel<float, 128, true>), grid, threads, lds, s, p);
      else hipLaunchKernelGGL((topk_attend_kernel<float, 128, false>), grid, threads, lds, s, p);
    } else {
      if (dec) hipLaunchKernelGGL((topk_attend_kernel<float, 64, true>), grid, threads, lds, s, p);
      else hipLaunchKernelGGL((topk_attend_kernel<float, 64, false>), grid, threads, lds, s, p);
    }
  }
  return hipGetLastError();
}

}  // namespace rat
