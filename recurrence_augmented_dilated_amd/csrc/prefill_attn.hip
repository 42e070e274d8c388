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
// bf16 kernel.  Block = 8 waves x 32 queries.  Per 64-key tile each wave
// computes S^T = K Q^T on v_mfma_f32_32x32x16_bf16 (keys on M, queries on N),
// so that after the online softmax its fp32 accumulators, converted to bf16,
// are already the B operand of O^T = V^T P^T: no shuffles between the two
// products.  Tiles stream through a four-stage LDS ring filled by direct
// global->LDS loads: K rows with XOR-swizzled 16-byte chunks, V from the
// scan's transposed layout, where one lane's eight keys of a 16-key step are
// a single 16-byte chunk; load addresses are a wave-uniform base plus a
// 32-bit lane offset.  Softmax runs in base 2 with the scale folded into one
// FMA, a v_maximum3 max tree, a lazily raised running max (the O rescale is
// rare) and row sums taken by v_dot2 over the same bf16 weights that enter
// P V.  Block order: dilation classes densest first, within a class the
// heaviest q-tile first with each (b, h) pair kept on one XCD.  A dense head
// with a window reads its grid from the all-state arrays (no second copy).
// The output rows go through the idle K ring and out as whole rows.
//
// fp32 kernel.  A plain exact-fp32 path (one or two lanes per query, keys
// staged in LDS) for fp32 inputs.
#include <algorithm>

#include "kv_stream.h"
#include "rat_internal.h"

namespace rat {
namespace {

constexpr int kWaves = 8;     // waves per block (bf16 kernel), 32 queries each
constexpr int kBM = 32 * kWaves;  // queries per block
constexpr int kBN = 64;       // keys per tile

struct AttnArgs {
  const void* q;
  void* out;
  const void* grid_k;
  const void* grid_v;
  const void* all_k;
  const void* all_v;
  int B, T, H, W;
  int64_t tpad;               // row length of the transposed all-states V
  int p0;                     // absolute position of query row 0
  int base;                   // absolute position of all-state row 0 (multiple of 64)
  int64_t arows;              // rows of the token-layout all-state buffers
  int n_qtiles;
  float sl2;                  // softmax scale * log2(e)
  HeadTable heads;            // dilation; grid keys at goff / gcap
  int64_t vgoff[kMaxHeads];   // grid values: element offset B * vgoff[h] * Dh
  int32_t vgcap[kMaxHeads];   // grid values: capacity (row length in kGridHeadCol)
  const int32_t* sel;         // block-selection mode: chosen blocks [B][T][H][sel_k]
  int sel_k;
  // dilation classes, densest first: class c holds heads hord[cls_h0[c] ..
  // cls_h0[c + 1]) and blocks [cls_b0[c], cls_b0[c + 1])
  int ncls;
  int cls_h0[kMaxCls + 1];
  int cls_b0[kMaxCls + 1];
  alignas(4) uint8_t hord[kMaxHeads];
};
static_assert(sizeof(AttnArgs) <= 4096, "kernel argument size");

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

// Work item -> (b, h, q-tile) over the dilation classes: a class's blocks run
// before those of sparser heads, so the heads whose key sets outgrow an XCD's
// L2 have their q-tiles in flight together and stream the same keys; within a
// class block_coords applies.  Every class but the last is padded to a
// multiple of 8 blocks, which keeps its XCD pinning; padding blocks get false.
__device__ __forceinline__ bool attn_block(const AttnArgs& a, int bid, int& b, int& h, int& qtile) {
  int c = 0;
  while (c + 1 < a.ncls && bid >= a.cls_b0[c + 1]) ++c;
  const int nh = a.cls_h0[c + 1] - a.cls_h0[c];
  const int rel = bid - a.cls_b0[c];
  if (rel >= a.B * nh * a.n_qtiles) return false;
  int hi;
  block_coords(rel, a.B, nh, a.n_qtiles, b, hi, qtile);
  // the byte of hord, read as its (scalar-loadable) dword
  const int i = a.cls_h0[c] + hi;
  h = int((reinterpret_cast<const uint32_t*>(a.hord)[i >> 2] >> (8 * (i & 3))) & 0xffu);
  return true;
}


// ---------------------------------------------------------------------------
// bf16 MFMA kernel
// ---------------------------------------------------------------------------

// v_permlane32_swap with both operands v: afterwards every lane holds the
// value of its column's lower-half lane (lane & 31) in lo and of its upper-half
// lane (lane | 32) in hi, without an LDS round trip.
__device__ __forceinline__ void half_pair(float v, float& lo, float& hi) {
  const uint32_t u = __float_as_uint(v);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  lo = __uint_as_float(r[0]);
  hi = __uint_as_float(r[1]);
}

// Max of a lane's 32 scores as a v_maximum3 tree (IEEE maximum: no
// canonicalising copies of the inputs, short dependency chains).
__device__ __forceinline__ float tree_max32(const floatx16_t* s) {
  auto mx = [](float x, float y) { return __builtin_elementwise_maximum(x, y); };
  float t[11];
#pragma unroll
  for (int i = 0; i < 10; ++i) {
    const int e0 = 3 * i, e1 = 3 * i + 1, e2 = 3 * i + 2;
    t[i] = mx(mx(s[e0 >> 4][e0 & 15], s[e1 >> 4][e1 & 15]), s[e2 >> 4][e2 & 15]);
  }
  t[10] = mx(s[1][14], s[1][15]);
  const float u0 = mx(mx(t[0], t[1]), t[2]);
  const float u1 = mx(mx(t[3], t[4]), t[5]);
  const float u2 = mx(mx(t[6], t[7]), t[8]);
  const float u3 = mx(t[9], t[10]);
  return mx(mx(u0, u1), mx(u2, u3));
}

// Lazy running max (base-2 units): a row's max moves only when a tile holds a
// score above it by more than kLazy, so every exp2 argument stays <= kLazy
// and the O rescale is rare.  The final division by the sum taken against the
// same max makes the result independent of this choice up to rounding.
constexpr float kLazy = 8.f;

typedef __attribute__((address_space(3))) void lds_void_t;
typedef const __attribute__((address_space(1))) void gbl_void_t;

// 16 bytes per lane straight from global memory at base + voff (a
// wave-uniform base in an SGPR pair plus a 32-bit per-lane byte offset) into
// LDS: lane l of the wave writes dst + 16 * l (dst must be wave-uniform).
// Written as asm so that the compiler does not treat every later LDS read as
// dependent on it (it cannot prove the ring stages disjoint and would wait
// for all loads in flight); the instruction has no destination register, and
// the kernel waits on vmcnt itself before a stage is read.
__device__ __forceinline__ void load_lds16(const void* base, uint32_t voff, void* dst) {
  const uint32_t lds = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_void_t*)dst));
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(lds), "v"(voff), "s"(base) : "memory");
}

// Wait until at most N of this wave's vector-memory operations are pending
// (vmcnt is six bits: the low four in bits 3:0, the high two in bits 15:14).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// The same for a run-time, wave-uniform bound n: waits for the largest
// multiple of G (at most 8 G) that does not exceed n, which is at least as
// long as a wait for n itself.
template <int G>
__device__ __forceinline__ void wait_vmcnt_atmost(int n) {
  if (n == G) wait_vmcnt<G>();
  else if (n >= 8 * G) wait_vmcnt<8 * G>();
  else if (n >= 7 * G) wait_vmcnt<7 * G>();
  else if (n >= 6 * G) wait_vmcnt<6 * G>();
  else if (n >= 5 * G) wait_vmcnt<5 * G>();
  else if (n >= 4 * G) wait_vmcnt<4 * G>();
  else if (n >= 3 * G) wait_vmcnt<3 * G>();
  else if (n >= 2 * G) wait_vmcnt<2 * G>();
  else if (n >= G) wait_vmcnt<G>();
  else wait_vmcnt<0>();
}

// Ring barrier: this wave's LDS reads are complete, then all waves meet.  A
// bare s_barrier (no release fence: that would also drain the prefetches in
// flight); the empty asm statements keep the compiler from moving memory
// accesses across it.
__device__ __forceinline__ void ring_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// SEL: block-selection key set (top-k block attention): block 0, the query's
// own block and its chosen blocks, 64 positions per block = one tile; the
// per-query lists sit in LDS and every lane walks its query's list as the
// block index grows.
template <int DH, bool SEL>
__global__ __launch_bounds__(kWaves * 64, 2) void attn_bf16_kernel(const AttnArgs a) {
  constexpr int KS = DH / 16;                 // MFMA k-steps over the head dim
  constexpr int DB = DH / 32;                 // 32-wide d blocks of O^T
  constexpr int KROW = DH * 2;                // bytes per K row
  constexpr int LPR = KROW / 16;              // lanes per K row in a direct load
  constexpr int KBYTES = kBN * KROW;          // K tile
  constexpr int VBYTES = DH * kBN * 2;        // V^T tile: DH rows of 64 keys
  constexpr int KL = KBYTES / 1024 / kWaves;  // direct loads per wave per tile
  constexpr int VL = VBYTES / 1024 / kWaves;
  static_assert(KL >= 1 && VL >= 1 && KL * kWaves * 1024 == KBYTES && VL * kWaves * 1024 == VBYTES, "tiles");

  // Four-stage ring: while tile it is consumed, tiles it+1..it+3 are landing
  // or in flight.
  __shared__ __attribute__((aligned(1024))) char sK[4][KBYTES];
  __shared__ __attribute__((aligned(1024))) char sV[4][VBYTES];

  int b, h, qtile;
  if (!attn_block(a, blockIdx.x, b, h, qtile)) return;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 31;
  const int g = lane >> 5;
  const int T = a.T, H = a.H, W = a.W;
  const int D = a.heads.dil[h];
  const int64_t rowC = (int64_t)H * DH;   // elements between tokens

  // query rows are relative to the call, key positions absolute (p0 + row)
  const int P0 = a.p0;
  const int t0 = qtile * kBM;
  const int t_last = min(t0 + kBM, T) - 1;
  const int tq = t0 + wave * 32 + n;      // this lane's query row (column of S^T)
  const bool q_live = tq < T;
  const int tqa = P0 + tq;                // its absolute position

  // Q^T fragments (B operand): query tq, head dims 16*ks + 8*g .. +7.  The
  // wave's 32 query rows are loaded as whole rows (64 / (DH / 8) rows per
  // instruction) into its part of the still idle K ring, 16-byte chunks
  // XOR-swizzled by row, and read back in fragment order; a barrier then
  // frees the ring for the first tiles.
  bf16x8_t qf[KS];
  {
    constexpr int CPR = DH / 8;     // 16-byte chunks per row
    constexpr int RPI = 64 / CPR;   // rows per load instruction
    char* qs = &sK[0][0] + wave * (32 * DH * 2);
    const bf16_t* qb = static_cast<const bf16_t*>(a.q) + (int64_t)b * T * rowC + h * DH + 8 * (lane % CPR);
    // rows past T read row T-1 (all loads in flight at once) and store zeros
    uint4 wq[32 / RPI];
#pragma unroll
    for (int i = 0; i < 32 / RPI; ++i) {
      const int row = t0 + wave * 32 + i * RPI + lane / CPR;
      wq[i] = *reinterpret_cast<const uint4*>(qb + (int64_t)min(row, T - 1) * rowC);
    }
#pragma unroll
    for (int i = 0; i < 32 / RPI; ++i) {
      const int r = i * RPI + lane / CPR, p = lane % CPR;
      const uint4 w = t0 + wave * 32 + r < T ? wq[i] : make_uint4(0, 0, 0, 0);
      *reinterpret_cast<uint4*>(qs + r * (DH * 2) + ((p ^ (r & (CPR - 1))) << 4)) = w;
    }
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): this wave's rows are in LDS
    asm volatile("" ::: "memory");
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qf[ks] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(
                                                 qs + n * (DH * 2) + (((2 * ks + g) ^ (n & (CPR - 1))) << 4)));
    ring_barrier();   // every wave has its fragments before the ring is filled
  }

  // key ranges of the block (window tiles start on a 64-key boundary)
  const int ng_hi = n_grid(P0 + t_last, W, D);
  const int ng_me = q_live ? n_grid(tqa, W, D) : 0;
  const int ntile_g = (ng_hi + kBN - 1) / kBN;
  const int j_lo = W > 0 ? max(a.base, P0 + t0 - W + 1) / kBN * kBN : 0;
  const int ntile_w = W > 0 ? (P0 + t_last - j_lo) / kBN + 1 : 0;
  const int ntiles = ntile_g + ntile_w;
  const int win_lo_me = max(0, tqa - W + 1);
  // this wave's queries (absolute): tiles that are fully masked for it are skipped
  const int tw0 = P0 + t0 + wave * 32;
  const int tw1 = P0 + min(t0 + wave * 32 + 31, T - 1);
  const bool wave_live = t0 + wave * 32 < T;
  const int ng_w0 = wave_live ? n_grid(tw0, W, D) : 0;
  const int ng_w1 = wave_live ? n_grid(tw1, W, D) : 0;

  const bf16_t* ak = W > 0 ? static_cast<const bf16_t*>(a.all_k) + (int64_t)b * a.arows * rowC + h * DH : nullptr;
  const bf16_t* avt = W > 0 ? static_cast<const bf16_t*>(a.all_v) + ((int64_t)b * H + h) * DH * a.tpad : nullptr;
  // A dense head with a window may have no stored grid (capacity 0): with
  // D = 1 and the all-state rows starting at position 0, grid entry i is
  // all-state row i, read in the window's layouts.
  const bool galias = !SEL && W > 0 && a.vgcap[h] == 0;
  // row length of the transposed grid values; in block-selection mode the
  // values are kAllHeadCol rows of tpad columns
  const int cap = SEL || galias ? int(a.tpad) : a.vgcap[h];
  const bf16_t* gk = galias ? ak : static_cast<const bf16_t*>(a.grid_k) + grid_row_offset(a.heads, a.B, b, h, 0, DH);
  const bf16_t* gvt = galias ? avt : static_cast<const bf16_t*>(a.grid_v) +
                      (SEL ? ((int64_t)b * H + h) * DH * a.tpad : ((int64_t)a.B * a.vgoff[h] + (int64_t)b * cap) * DH);

  // issue the direct loads of tile `it` into (dK, dV)
  // per-lane parts of the direct-load addresses (bytes): K row within the
  // tile and its chunk; V^T row (grid and window layouts) and chunk
  int k_row[KL];
  uint32_t k_chunk[KL], v_off_g[VL], v_off_w[VL];
#pragma unroll
  for (int u = 0; u < KL; ++u) {
    const int j = wave * KL + u;                 // 1 KB slice of the tile
    const int r = j * (64 / LPR) + lane / LPR;   // key row
    const int p = lane % LPR;                    // physical 16-byte chunk
    k_row[u] = r;
    k_chunk[u] = 16u * uint32_t(p ^ (r & (LPR - 1) & 15));   // logical chunk stored there
  }
#pragma unroll
  for (int u = 0; u < VL; ++u) {
    const int j = wave * VL + u;
    const uint32_t d = uint32_t(j * 8 + lane / 8);             // head-dim row of V^T
    v_off_g[u] = d * uint32_t(cap) * 2u + 16u * uint32_t(lane % 8);
    v_off_w[u] = W > 0 ? d * uint32_t(a.tpad) * 2u + 16u * uint32_t(lane % 8) : 0u;
  }
  const uint32_t krow_w = uint32_t(rowC) * 2u, krow_g = galias ? krow_w : DH * 2;   // K row strides (bytes)

  // issue the direct loads of tile `it` into (dK, dV); the tile's first row
  // goes into the wave-uniform base, rows past the last valid one re-read it
  auto issue = [&](int it, char* dK, char* dV) __attribute__((always_inline)) {
    const bool isg = it < ntile_g;
    const int row0 = isg ? it * kBN : j_lo + (it - ntile_g) * kBN - a.base;   // buffer row of the tile
    const int nvalid = isg ? ng_hi - row0 : P0 + t_last + 1 - (row0 + a.base);
    const uint32_t krow = isg ? krow_g : krow_w;
    const char* kb = reinterpret_cast<const char*>(isg ? gk : ak) + (int64_t)row0 * krow;
    const char* vb = reinterpret_cast<const char*>(isg ? gvt : avt) + (int64_t)row0 * 2;
#pragma unroll
    for (int u = 0; u < KL; ++u)
      load_lds16(kb, uint32_t(min(k_row[u], nvalid - 1)) * krow + k_chunk[u], dK + (wave * KL + u) * 1024);
#pragma unroll
    for (int u = 0; u < VL; ++u) {
      const uint32_t og = v_off_g[u], ow = v_off_w[u];
      load_lds16(vb, isg ? og : ow, dV + (wave * VL + u) * 1024);
    }
  };

  // per-lane byte offsets of the V^T fragments in a tile: the chunk of
  // 16-key step st for head-dim rows 32 db + n depends on db only through its
  // parity (rows 64 apart share the swizzle), so eight offsets serve all
  // (st, db), the rest is an immediate
  uint32_t vo[4][2];
#pragma unroll
  for (int st = 0; st < 4; ++st)
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int d = 32 * p + n;
      vo[st][p] = uint32_t(d * (kBN * 2) + 16 * ((2 * st + g) ^ col_swz(d)));
    }
  auto v_at = [&](const char* cV, int st, int db) __attribute__((always_inline)) -> uint4 {
    return *reinterpret_cast<const uint4*>(cV + vo[st][db & 1] + (db >> 1) * (64 * kBN * 2));
  };

  floatx16_t o[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[i][r] = 0.f;
  float m_run = -INFINITY;
  float l_run = 0.f;

  // needed: does any query of this wave see a key of tile it?
  // masked: does some (query, key) pair of the tile fall outside the key set?
  // block-selection mode: is block it in this lane's query's key set
  constexpr int kSelStride = kSelMaxK + 1;   // list entries plus a -1 sentinel
  __shared__ int32_t s_sel[SEL ? kBM * kSelStride : 1];
  bool lane_sel = true;
  int sel_ptr = 0, sel_nxt = -1;
  const int sel_row = (wave * 32 + n) * kSelStride;
  const int own_blk = tqa / kBN;
  auto sel_advance = [&](int it) __attribute__((always_inline)) {
    const bool hit = sel_nxt == it;
    lane_sel = (it == 0) | (it == own_blk) | hit;
    sel_ptr += hit ? 1 : 0;
    sel_nxt = s_sel[sel_row + sel_ptr];
  };

  auto tile_info = [&](int it, bool& is_grid, bool& needed, bool& masked, int& kbase) __attribute__((always_inline)) {
    is_grid = it < ntile_g;
    if (SEL) {
      // grid tiles only (D = 1, W = 0); skip a tile no query of the wave
      // keeps, mask it unless every query keeps it
      kbase = it * kBN;
      const uint64_t keep = __ballot(lane_sel && q_live && kbase < ng_me);
      needed = keep != 0;
      masked = kbase + kBN > ng_w0 || keep != __ballot(q_live);
    } else if (is_grid) {
      kbase = it * kBN;
      needed = wave_live && kbase < ng_w1;
      masked = kbase + kBN > ng_w0;
    } else {
      kbase = j_lo + (it - ntile_g) * kBN;
      needed = wave_live && kbase <= tw1 && kbase + kBN - 1 >= max(0, tw0 - W + 1);
      masked = !(kbase >= tw1 - W + 1 && kbase + kBN - 1 <= tw0);
    }
  };

  // S^T = K Q^T of one tile into sc (two 32-key blocks)
  auto scores = [&](const char* cK, floatx16_t* sc) __attribute__((always_inline)) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) sc[kb][r] = 0.f;
    // the two 32-key chains interleaved; each K read leads its MFMA by
    // several others
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const int m = 32 * kb + n;
        const int c = (2 * ks + g) ^ (m & (LPR - 1) & 15);
        const uint4 w = *reinterpret_cast<const uint4*>(cK + m * KROW + 16 * c);
        sc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, w), qf[ks], sc[kb], 0, 0, 0);
      }
    constexpr int NM = 2 * KS, LEAD = 6;
#pragma unroll
    for (int i = 0; i < LEAD; ++i) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
#pragma unroll
    for (int i = 0; i < NM; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (i + LEAD < NM) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
  };

  // mask, online softmax and O^T += V^T P^T for the scores s of tile it
  auto finish = [&](int it, const char* cV, floatx16_t* s) __attribute__((always_inline)) {
    bool is_grid, needed, masked;
    int kbase;
    tile_info(it, is_grid, needed, masked, kbase);
    if (!needed) return;
    // ---- mask: key index kbase + c(kb, r) + 4g, branch-free selects
    if (masked) {
      // key kbase + 4g + c is valid iff lo <= c <= hi: grid keys below this
      // query's count, window keys in [max(0, t-W+1), t]; one unsigned
      // range compare per score
      const int key0 = kbase + 4 * g;
      const int lo = is_grid ? -64 : win_lo_me - key0;
      const int hi = is_grid ? ng_me - 1 - key0 : tqa - key0;
      const bool none = hi < lo || !lane_sel;
      const int lo2 = none ? 1 << 20 : lo;
      const uint32_t span = none ? 0u : uint32_t(hi - lo);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int c = 32 * kb + 8 * (r >> 2) + (r & 3);
          s[kb][r] = uint32_t(c - lo2) <= span ? s[kb][r] : -INFINITY;
        }
    }

    // V^T fragments of the first two 16-key steps, read before the softmax
    // so that their latency hides under it
    uint4 vpre[2 * DB];
#pragma unroll
    for (int j = 0; j < 2 * DB; ++j) {
      vpre[j] = v_at(cV, j / DB, j % DB);
    }

    // ---- online softmax (base 2; running max shared by the two lane halves)
    float mx_lo, mx_hi;
    half_pair(tree_max32(s), mx_lo, mx_hi);
    const float mt = __builtin_elementwise_maximum(mx_lo, mx_hi) * a.sl2;
    const bool up = mt > m_run + kLazy;
    if (__ballot(up) != 0) {
      const float m_new = up ? mt : m_run;
      const float alpha = up ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.f;
      l_run *= alpha;
#pragma unroll
      for (int i = 0; i < DB; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[i][r] *= alpha;
      m_run = m_new;
    }
    const float nm = m_run == -INFINITY ? 0.f : -m_run;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) s[kb][r] = __builtin_amdgcn_exp2f(fmaf(s[kb][r], a.sl2, nm));

    // ---- bf16 P^T fragments; row sums over the same rounded weights
    uint4 pws[4];
    float lp0 = 0.f, lp1 = 0.f;
    const bf16x2_t ones = __builtin_bit_cast(bf16x2_t, 0x3f803f80u);
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      const int kb = st >> 1;
      const int r0 = 8 * (st & 1);
      pws[st].x = pack_bf16x2(s[kb][r0 + 0], s[kb][r0 + 1]);
      pws[st].y = pack_bf16x2(s[kb][r0 + 2], s[kb][r0 + 3]);
      pws[st].z = pack_bf16x2(s[kb][r0 + 4], s[kb][r0 + 5]);
      pws[st].w = pack_bf16x2(s[kb][r0 + 6], s[kb][r0 + 7]);
      lp0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pws[st].x), ones, lp0, false);
      lp1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pws[st].y), ones, lp1, false);
      lp0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pws[st].z), ones, lp0, false);
      lp1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pws[st].w), ones, lp1, false);
    }
    l_run += lp0 + lp1;
    // ---- O^T += V^T P^T over four 16-key steps
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      const bf16x8_t pf = __builtin_bit_cast(bf16x8_t, pws[st]);
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        // keys 16st + 4g + {0..3} and 16st + 8 + 4g + {0..3}: one 16-byte chunk
        const uint4 vw = st < 2 ? vpre[st * DB + db] : v_at(cV, st, db);
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, vw), pf, o[db], 0, 0, 0);
      }
    }
  };

  constexpr int LPW = KL + VL;   // direct loads per wave per tile
  constexpr int kAhead = 3;      // tiles in flight ahead of the one consumed
  floatx16_t sc[2];
  // Tile it in ring slot S (= it & 3), a compile-time constant: every LDS
  // read then addresses a per-lane base plus an immediate offset.
  using Slot0 = std::integral_constant<int, 0>;
  using Slot1 = std::integral_constant<int, 1>;
  using Slot2 = std::integral_constant<int, 2>;
  using Slot3 = std::integral_constant<int, 3>;

  wait_vmcnt<0>();   // Q fragments are in registers before the ring starts
  if (W > 0) {
    // With a window band every wave skips some of the block's window tiles,
    // so tiles go in pairs between barriers: while pair p is consumed, pair
    // p+1 lands in the other half of the ring (the slots of pair p-1, free
    // since the last barrier), and a wave that skips one tile of a pair goes
    // straight on to the other.
    for (int p = 0; p < 2 && p < ntiles; ++p) issue(p, sK[p], sV[p]);
    if (ntiles > 0) {
      wait_vmcnt<0>();
      ring_barrier();
    }
    auto pair = [&](int t0, auto SA, auto SB) __attribute__((always_inline)) {
      constexpr int sa = decltype(SA)::value;
      constexpr int sb = decltype(SB)::value;
      // the next pair goes into the slots of the previous one
      // each tile of the next pair goes out once a tile of this pair has
      // its products under way
      auto tile_then = [&](int it, auto S, int nxt, char* dK, char* dV) __attribute__((always_inline)) {
        constexpr int slot = decltype(S)::value;
        bool is_grid, needed, masked;
        int kbase;
        tile_info(it, is_grid, needed, masked, kbase);
        if (needed) scores(sK[slot], sc);
        if (nxt < ntiles) issue(nxt, dK, dV);
        if (needed) finish(it, sV[slot], sc);
      };
      tile_then(t0, SA, t0 + 2, sK[sa ^ 2], sV[sa ^ 2]);
      if (t0 + 1 < ntiles) tile_then(t0 + 1, SB, t0 + 3, sK[sb ^ 2], sV[sb ^ 2]);
      wait_vmcnt<0>();
      ring_barrier();
    };
    for (int t0 = 0; t0 < ntiles; t0 += 4) {
      pair(t0, Slot0{}, Slot1{});
      if (t0 + 2 < ntiles) pair(t0 + 2, Slot2{}, Slot3{});
    }
  } else {
    if constexpr (SEL) {
      // the block's chosen lists into LDS (made visible by the barrier below)
      for (int e = tid; e < kBM * kSelStride; e += kWaves * 64) {
        const int qi = e / kSelStride, j = e - qi * kSelStride;
        const int tr = t0 + qi;
        s_sel[e] = (j < a.sel_k && tr < T) ? a.sel[(((int64_t)b * T + tr) * H + h) * a.sel_k + j] : -1;
      }
      wait_vmcnt<0>();
    }
    // one tile per barrier, three in flight
    for (int p = 0; p < kAhead && p < ntiles; ++p) issue(p, sK[p], sV[p]);
    if (ntiles > 0) {
      const int later = min(ntiles, kAhead) - 1;   // tiles issued after tile 0
      if (later >= 2) wait_vmcnt<2 * LPW>();
      else if (later == 1) wait_vmcnt<LPW>();
      else wait_vmcnt<0>();
      ring_barrier();
    }
    if constexpr (SEL) sel_nxt = s_sel[sel_row];
    auto step = [&](int it, auto S) __attribute__((always_inline)) {
      constexpr int slot = decltype(S)::value;
      // tile it + kAhead goes into the slot of tile it - 1
      if constexpr (SEL) sel_advance(it);
      {
        bool is_grid, needed, masked;
        int kbase;
        tile_info(it, is_grid, needed, masked, kbase);
        if (needed) scores(sK[slot], sc);
        // the loads of tile it + kAhead go out once this tile's products are
        // under way (issued right after the barrier, the block's 32 loads
        // queue ahead of every wave's first MFMA)
        if (it + kAhead < ntiles) issue(it + kAhead, sK[(slot + kAhead) & 3], sV[(slot + kAhead) & 3]);
        if (needed) finish(it, sV[slot], sc);
      }
      // tile it+1 must have landed; later tiles may still fly
      const int later = min(ntiles - 1, it + kAhead) - (it + 1);
      if (later >= 2) wait_vmcnt<2 * LPW>();
      else if (later == 1) wait_vmcnt<LPW>();
      else wait_vmcnt<0>();
      ring_barrier();
    };
    for (int it = 0; it < ntiles; it += 4) {
      step(it, Slot0{});
      if (it + 1 < ntiles) step(it + 1, Slot1{});
      if (it + 2 < ntiles) step(it + 2, Slot2{});
      if (it + 3 < ntiles) step(it + 3, Slot3{});
    }
  }

  // ---- normalise and store (empty key set -> zeros).  Every loop path
  // ends with its loads waited for and a ring barrier, so the K ring is idle:
  // each wave stages its 32 output rows in its own part of it (row-major,
  // 16-byte chunks XOR-swizzled by row) and writes whole rows with 16-byte
  // stores, one instruction covering 64 / (DH / 8) complete rows.
  float l_lo, l_hi;
  half_pair(l_run, l_lo, l_hi);
  const float l_tot = l_lo + l_hi;
  const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
  constexpr int CPR = DH / 8;     // 16-byte chunks per output row
  constexpr int RPI = 64 / CPR;   // rows per store instruction
  static_assert(kWaves * 32 * DH * 2 == 4 * KBYTES, "the output rows fill the K ring");
  char* ep = &sK[0][0] + wave * (32 * DH * 2);
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int k4 = 0; k4 < 4; ++k4) {
      const int c = 4 * db + k4;   // chunk of head dims 32 db + 8 k4 .. +7; this lane's half is g
      const uint2 w = make_uint2(pack_bf16x2(o[db][4 * k4 + 0] * inv, o[db][4 * k4 + 1] * inv),
                                 pack_bf16x2(o[db][4 * k4 + 2] * inv, o[db][4 * k4 + 3] * inv));
      *reinterpret_cast<uint2*>(ep + n * (DH * 2) + ((c ^ (n & (CPR - 1))) << 4) + 8 * g) = w;
    }
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): this wave's rows are in LDS
  asm volatile("" ::: "memory");
  bf16_t* ob = static_cast<bf16_t*>(a.out) + ((int64_t)b * T + t0 + wave * 32) * rowC + h * DH;
#pragma unroll
  for (int i = 0; i < 32 / RPI; ++i) {
    const int r = i * RPI + lane / CPR;   // row of the wave's 32
    const int p = lane % CPR;             // physical chunk
    const uint4 w = *reinterpret_cast<const uint4*>(ep + r * (DH * 2) + (p << 4));
    if (t0 + wave * 32 + r < T)
      *reinterpret_cast<uint4*>(ob + (int64_t)r * rowC + ((p ^ (r & (CPR - 1))) << 3)) = w;
  }
}

// ---------------------------------------------------------------------------
// bf16 MFMA kernel, persistent form for grid-only key sets (W = 0)
// ---------------------------------------------------------------------------
//
// One block per compute unit walks a list of q-tiles (the work items of the
// one-block-per-q-tile launch) and streams their 64-key tiles through one
// three-slot ring as if they were one sequence: the next q-tile's Q rows and
// first tiles load while the current q-tile's last tiles are computed, so no
// block start, Q landing or first-tile wait sits between q-tiles.  The tile
// math is that of attn_bf16_kernel.  Each wave owns a staging area for its
// 32 query rows: the next q-tile's Q rows land there by direct loads while
// the current q-tile runs and are read into fragments once its last tile's
// scores are taken (the old fragments are dead then); the current q-tile's
// output rows are staged there after that and stored as whole rows at the
// start of the next step, under that step's work.  The Q rows of the q-tile
// after the next wait until the area is free again, so the loads run at most
// one q-tile ahead.  q-tiles whose rows have no key get their zero rows when
// the list reaches them.
//
// Item order: within an XCD (blocks and items are dealt to the XCDs by index
// mod 8, which keeps every (b, h) pair on one XCD as in the plain launch) the
// heaviest-first item list is cut into rounds of one item per block, dealt
// ascending in even rounds and descending in odd ones, which evens out the
// per-block sums of a list whose costs fall steadily.
//
// Waits: this wave's loads complete in issue order, so a tile has landed once
// at most as many vector-memory operations are pending as loads were issued
// after it.  Stores are never counted: a pending store only makes such a wait
// longer, whatever the order in which stores complete.
constexpr int kPSlots = 3;   // one tile consumed, two in flight

struct StreamItem {
  int b, h, t0, ntiles;
};
struct StreamSrc {   // where an item's tiles come from
  const char* gk;    // grid keys of (b, h), row-major
  const char* gvt;   // grid values of (b, h), transposed
  int ng_hi, cap;
};

// A copy of x that the compiler must treat as new: values derived from it
// are recomputed where they are used instead of being hoisted out of the
// loop and kept live (or spilled) across it.
__device__ __forceinline__ uint32_t opaque_s(uint32_t x) {
  asm volatile("" : "+s"(x));
  return x;
}
__device__ __forceinline__ uint32_t opaque_v(uint32_t x) {
  asm volatile("" : "+v"(x));
  return x;
}
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((const lds_void_t*)p));
}
// load_lds16 with the LDS address given as a number
__device__ __forceinline__ void load_lds16_to(const void* base, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(lds), "v"(voff), "s"(base) : "memory");
}

template <int DH>
__global__ __launch_bounds__(kWaves * 64, 2) void attn_bf16_stream_kernel(const AttnArgs a) {
  constexpr int KS = DH / 16;
  constexpr int DB = DH / 32;
  constexpr int KROW = DH * 2;
  constexpr int LPR = KROW / 16;
  constexpr int KBYTES = kBN * KROW;
  constexpr int VBYTES = DH * kBN * 2;
  constexpr int KL = KBYTES / 1024 / kWaves;
  constexpr int VL = VBYTES / 1024 / kWaves;
  constexpr int LPW = KL + VL;       // direct loads per wave per tile
  constexpr int CPR = DH / 8;        // 16-byte chunks per query / output row
  constexpr int RPI = 64 / CPR;      // rows per load / store instruction
  constexpr int QL = 32 / RPI;       // instructions for a wave's 32 rows
  constexpr int AREA = 32 * KROW;    // a wave's staging area
  static_assert(KL >= 1 && VL >= 1 && KL * kWaves * 1024 == KBYTES && VL * kWaves * 1024 == VBYTES, "tiles");
  static_assert(QL * 1024 == AREA, "staging area");
  constexpr int G = QL < LPW ? QL : LPW;   // every load count is a multiple of G
  static_assert(QL % G == 0 && LPW % G == 0, "load counts");

  __shared__ __attribute__((aligned(1024))) char sK[kPSlots][KBYTES];
  __shared__ __attribute__((aligned(1024))) char sV[kPSlots][VBYTES];
  __shared__ __attribute__((aligned(1024))) char sA[kWaves][AREA];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 31;
  const int g = lane >> 5;
  const int T = a.T;
  const int64_t rowC = (int64_t)a.H * DH;
  const int P0 = a.p0;
  char* const wa = sA[wave];

  // ---- the block's items
  const int nb = a.cls_b0[a.ncls];
  const int xcd = blockIdx.x & 7;
  const int li = blockIdx.x >> 3;
  const int nbx = gridDim.x >> 3;                  // blocks per XCD
  const int nrounds = ((nb + 7) / 8 + nbx - 1) / nbx;
  auto item_at = [&](int r, StreamItem& it) __attribute__((always_inline)) -> bool {
    const int k = r * nbx + ((r & 1) ? nbx - 1 - li : li);
    const int bid = 8 * k + xcd;
    int qtile;
    if (bid >= nb || !attn_block(a, bid, it.b, it.h, qtile)) return false;
    it.t0 = qtile * kBM;
    it.ntiles = ((P0 + min(it.t0 + kBM, T)) / a.heads.dil[it.h] + kBN - 1) / kBN;
    return true;
  };
  auto src_of = [&](const StreamItem& it) __attribute__((always_inline)) -> StreamSrc {
    StreamSrc r;
    r.ng_hi = (P0 + min(it.t0 + kBM, T)) / a.heads.dil[it.h];   // grid entries of the last row
    r.cap = a.vgcap[it.h];
    r.gk = reinterpret_cast<const char*>(static_cast<const bf16_t*>(a.grid_k) +
                                         grid_row_offset(a.heads, a.B, it.b, it.h, 0, DH));
    r.gvt = reinterpret_cast<const char*>(static_cast<const bf16_t*>(a.grid_v) +
                                          ((int64_t)a.B * a.vgoff[it.h] + (int64_t)it.b * r.cap) * DH);
    return r;
  };
  // rows t0 + wave * 32 + r (r < 32) of head h; rows past T are not written
  auto out_rows = [&](const StreamItem& it) __attribute__((always_inline)) {
    return static_cast<bf16_t*>(a.out) + ((int64_t)it.b * T + it.t0 + wave * 32) * rowC + it.h * DH;
  };
  // next item with keys after round r (r advances to it); items without keys
  // on the way get their zero rows
  auto advance = [&](int& r, StreamItem& it) __attribute__((always_inline)) -> bool {
    while (++r < nrounds) {
      if (!item_at(r, it)) continue;
      if (it.ntiles > 0) return true;
      bf16_t* ob = out_rows(it);
      const uint32_t l = opaque_v(uint32_t(lane));
#pragma unroll
      for (int i = 0; i < QL; ++i) {
        const uint32_t rr = i * RPI + l / CPR;
        if (it.t0 + wave * 32 + int(rr) < T)
          *reinterpret_cast<uint4*>(ob + __umul24(rr, uint32_t(rowC)) + 8 * (l % CPR)) = make_uint4(0, 0, 0, 0);
      }
    }
    return false;
  };

  // ---- direct loads
  // Q rows of the wave into its area: row r, physical chunk p holds logical
  // chunk p ^ (r mod CPR); rows past T re-read row T - 1
  auto issue_q = [&](const StreamItem& it) __attribute__((always_inline)) {
    const int r0 = min(it.t0 + wave * 32, T - 1);
    const uint32_t rmax = uint32_t(T - 1 - r0);
    const char* base = reinterpret_cast<const char*>(static_cast<const bf16_t*>(a.q) +
                                                     ((int64_t)it.b * T + r0) * rowC + it.h * DH);
    const uint32_t l = opaque_v(uint32_t(lane));
    const uint32_t q = l / CPR;                      // row within the instruction's RPI rows
    const uint32_t c0 = 16u * ((l % CPR) ^ q);       // its chunk, before the row's swizzle bits
    const uint32_t wb = opaque_s(lds_addr(wa));
#pragma unroll
    for (int i = 0; i < QL; ++i) {
      // row i * RPI + q: (i * RPI) mod CPR is a multiple of RPI > q, so the
      // row's swizzle is c0 ^ that
      const uint32_t r = min(uint32_t(i * RPI) + q, rmax);
      const uint32_t off = __umul24(r, uint32_t(rowC * 2)) + (c0 ^ (16u * uint32_t((i * RPI) & (CPR - 1))));
      load_lds16_to(base, off, wb + i * 1024);
    }
  };
  int k_row[KL];
  uint32_t k_chunk[KL], v_row2[VL];
#pragma unroll
  for (int u = 0; u < KL; ++u) {
    const int j = wave * KL + u;
    const int r = j * (64 / LPR) + lane / LPR;
    const int p = lane % LPR;
    k_row[u] = r;
    k_chunk[u] = 16u * uint32_t(p ^ (r & (LPR - 1) & 15));
  }
#pragma unroll
  for (int u = 0; u < VL; ++u) v_row2[u] = 2u * uint32_t((wave * VL + u) * 8 + lane / 8);
  const uint32_t v_col = 16u * uint32_t(lane % 8);
  // tile t of the item whose source is src, into ring slot S
  auto issue_tile = [&](const StreamSrc& src, int t, auto Sc) __attribute__((always_inline)) {
    constexpr int S = decltype(Sc)::value;
    const int row0 = t * kBN;
    const int nvalid = src.ng_hi - row0;
    const char* kb = src.gk + (int64_t)row0 * KROW;
    const char* vb = src.gvt + (int64_t)row0 * 2;
    const uint32_t kd = opaque_s(lds_addr(sK[0]) + uint32_t(wave * KL * 1024));
    const uint32_t vd = opaque_s(lds_addr(sV[0]) + uint32_t(wave * VL * 1024));
#pragma unroll
    for (int u = 0; u < KL; ++u)
      load_lds16_to(kb, uint32_t(min(k_row[u], nvalid - 1)) * KROW + k_chunk[u], kd + S * KBYTES + u * 1024);
#pragma unroll
    for (int u = 0; u < VL; ++u)
      load_lds16_to(vb, v_row2[u] * uint32_t(src.cap) + v_col, vd + S * VBYTES + u * 1024);
  };

  uint32_t vo[4][2];
#pragma unroll
  for (int st = 0; st < 4; ++st)
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int d = 32 * p + n;
      vo[st][p] = uint32_t(d * (kBN * 2) + 16 * ((2 * st + g) ^ col_swz(d)));
    }
  auto v_at = [&](const char* cV, int st, int db) __attribute__((always_inline)) -> uint4 {
    return *reinterpret_cast<const uint4*>(cV + vo[st][db & 1] + (db >> 1) * (64 * kBN * 2));
  };

  // ---- consumer state of the current item
  bf16x8_t qf[KS];
  floatx16_t o[DB];
  float m_run, l_run;
  int ng_me, ng_w0, ng_w1;
  bool wave_live;
  auto enter = [&](const StreamItem& it) __attribute__((always_inline)) {
    const int D = a.heads.dil[it.h];
    const int tq = it.t0 + wave * 32 + n;
    ng_me = tq < T ? (P0 + tq + 1) / D : 0;
    wave_live = it.t0 + wave * 32 < T;
    ng_w0 = wave_live ? (P0 + it.t0 + wave * 32 + 1) / D : 0;
    ng_w1 = wave_live ? (P0 + min(it.t0 + wave * 32 + 31, T - 1) + 1) / D : 0;
#pragma unroll
    for (int i = 0; i < DB; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[i][r] = 0.f;
    m_run = -INFINITY;
    l_run = 0.f;
  };
  auto read_q = [&]() __attribute__((always_inline)) {
    const uint32_t l = opaque_v(uint32_t(lane));
    const uint32_t ln = l & 31, lg = l >> 5;
    const char* row = wa + ln * KROW;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qf[ks] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(
                                                row + (((2 * ks + lg) ^ (ln & (CPR - 1))) << 4)));
  };

  auto scores = [&](const char* cK, floatx16_t* sc) __attribute__((always_inline)) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) sc[kb][r] = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const int m = 32 * kb + n;
        const int c = (2 * ks + g) ^ (m & (LPR - 1) & 15);
        const uint4 w = *reinterpret_cast<const uint4*>(cK + m * KROW + 16 * c);
        sc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, w), qf[ks], sc[kb], 0, 0, 0);
      }
    constexpr int NM = 2 * KS, LEAD = 6;
#pragma unroll
    for (int i = 0; i < LEAD; ++i) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
#pragma unroll
    for (int i = 0; i < NM; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (i + LEAD < NM) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
  };

  auto finish = [&](int kbase, bool masked, const char* cV, floatx16_t* s) __attribute__((always_inline)) {
    if (masked) {
      // grid key kbase + 4g + c is valid iff c <= ng_me - 1 - kbase - 4g
      const int key0 = kbase + 4 * g;
      const int lo = -64;
      const int hi = ng_me - 1 - key0;
      const bool none = hi < lo;
      const int lo2 = none ? 1 << 20 : lo;
      const uint32_t span = none ? 0u : uint32_t(hi - lo);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int c = 32 * kb + 8 * (r >> 2) + (r & 3);
          s[kb][r] = uint32_t(c - lo2) <= span ? s[kb][r] : -INFINITY;
        }
    }
    uint4 vpre[2 * DB];
#pragma unroll
    for (int j = 0; j < 2 * DB; ++j) vpre[j] = v_at(cV, j / DB, j % DB);

    float mx_lo, mx_hi;
    half_pair(tree_max32(s), mx_lo, mx_hi);
    const float mt = __builtin_elementwise_maximum(mx_lo, mx_hi) * a.sl2;
    const bool up = mt > m_run + kLazy;
    if (__ballot(up) != 0) {
      const float m_new = up ? mt : m_run;
      const float alpha = up ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.f;
      l_run *= alpha;
#pragma unroll
      for (int i = 0; i < DB; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[i][r] *= alpha;
      m_run = m_new;
    }
    const float nm = m_run == -INFINITY ? 0.f : -m_run;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) s[kb][r] = __builtin_amdgcn_exp2f(fmaf(s[kb][r], a.sl2, nm));

    uint4 pws[4];
    float lp0 = 0.f, lp1 = 0.f;
    const bf16x2_t ones = __builtin_bit_cast(bf16x2_t, 0x3f803f80u);
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      const int kb = st >> 1;
      const int r0 = 8 * (st & 1);
      pws[st].x = pack_bf16x2(s[kb][r0 + 0], s[kb][r0 + 1]);
      pws[st].y = pack_bf16x2(s[kb][r0 + 2], s[kb][r0 + 3]);
      pws[st].z = pack_bf16x2(s[kb][r0 + 4], s[kb][r0 + 5]);
      pws[st].w = pack_bf16x2(s[kb][r0 + 6], s[kb][r0 + 7]);
      lp0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pws[st].x), ones, lp0, false);
      lp1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pws[st].y), ones, lp1, false);
      lp0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pws[st].z), ones, lp0, false);
      lp1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pws[st].w), ones, lp1, false);
    }
    l_run += lp0 + lp1;
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      const bf16x8_t pf = __builtin_bit_cast(bf16x8_t, pws[st]);
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const uint4 vw = st < 2 ? vpre[st * DB + db] : v_at(cV, st, db);
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, vw), pf, o[db], 0, 0, 0);
      }
    }
  };

  // normalised output rows of the current item into the wave's area
  // (row-major, chunks XOR-swizzled by row)
  auto stage = [&]() __attribute__((always_inline)) {
    float l_lo, l_hi;
    half_pair(l_run, l_lo, l_hi);
    const float l_tot = l_lo + l_hi;
    const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
    const uint32_t l = opaque_v(uint32_t(lane));
    const uint32_t ln = l & 31, lg = l >> 5;
    char* const row = wa + ln * KROW + 8 * lg;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int k4 = 0; k4 < 4; ++k4) {
        const uint32_t c = 4 * db + k4;
        const uint2 w = make_uint2(pack_bf16x2(o[db][4 * k4 + 0] * inv, o[db][4 * k4 + 1] * inv),
                                   pack_bf16x2(o[db][4 * k4 + 2] * inv, o[db][4 * k4 + 3] * inv));
        *reinterpret_cast<uint2*>(row + ((c ^ (ln & (CPR - 1))) << 4)) = w;
      }
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): the rows are in LDS
    asm volatile("" ::: "memory");
  };
  // the staged rows of item `it` out as whole rows; afterwards the area is free
  auto flush = [&](const StreamItem& it) __attribute__((always_inline)) {
    bf16_t* ob = out_rows(it);
    const uint32_t l2 = opaque_v(uint32_t(lane));
    const uint32_t q = l2 / CPR, p = l2 % CPR;
#pragma unroll
    for (int i = 0; i < QL; ++i) {
      const uint32_t r = i * RPI + q;
      const uint4 w = *reinterpret_cast<const uint4*>(wa + r * KROW + (p << 4));
      if (it.t0 + wave * 32 + int(r) < T)
        *reinterpret_cast<uint4*>(ob + __umul24(r, uint32_t(rowC)) + ((p ^ (r & (CPR - 1))) << 3)) = w;
    }
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);   // the area is read before it takes new Q rows
    asm volatile("" ::: "memory");
  };

  // ---- prologue: the first item's Q rows and up to two of its tiles
  StreamItem C, N;
  int rN = -1;
  if (!advance(rN, C)) return;
  bool hasN = advance(rN, N);
  enter(C);
  int loads = 0;              // direct loads this wave has issued (stores are not counted)
  int e[kPSlots] = {0, 0, 0};  // value of `loads` right after the tile in each slot was issued
  issue_q(C);
  loads += QL;
  StreamSrc I = src_of(C);    // the issue cursor's item (C, or N once C's tiles are out)
  int I_ntiles = C.ntiles;
  issue_tile(I, 0, std::integral_constant<int, 0>{});
  loads += LPW;
  e[0] = loads;
  int iss = 1;                // its next tile
  bool curN = false;          // the issue cursor is in N
  int qN = 0;                 // value of `loads` right after N's Q rows were issued
  int ahead = 0;              // tiles issued beyond the one being consumed
  if (C.ntiles > 1) {
    issue_tile(I, 1, std::integral_constant<int, 1>{});
    loads += LPW;
    e[1] = loads;
    iss = 2;
    ahead = 1;
  }
  wait_vmcnt_atmost<G>(loads - e[0]);   // Q rows and tile 0 have landed
  read_q();
  ring_barrier();

  // issue the next tile of the stream into slot S, if it exists and its
  // item is C or N; entering N first sends N's Q rows into the area (free
  // since C's Q rows were read and the previous output rows went out)
  auto issue_next = [&](auto Sc) __attribute__((always_inline)) -> bool {
    if (iss == I_ntiles) {
      if (curN || !hasN) return false;
      curN = true;
      I = src_of(N);
      I_ntiles = N.ntiles;
      iss = 0;
      issue_q(N);
      loads += QL;
      qN = loads;
    }
    constexpr int S = decltype(Sc)::value;
    issue_tile(I, iss++, Sc);
    loads += LPW;
    e[S] = loads;
    return true;
  };

  floatx16_t sc[2];
  int jt = 0;                 // tile of C in the slot being consumed
  bool done = false;
  // the previous item's output rows wait in the area until the next step
  // begins, so that their stores complete under that step's work instead of
  // lengthening the wait that ends this one
  StreamItem P = C;
  bool pend = false;
  auto step = [&](auto Sc) __attribute__((always_inline)) {
    constexpr int S = decltype(Sc)::value;
    constexpr int S1 = (S + 1) % kPSlots, S2 = (S + 2) % kPSlots;
    const int kbase = jt * kBN;
    const bool needed = wave_live && kbase < ng_w1;
    const bool masked = kbase + kBN > ng_w0;
    if (pend) {
      flush(P);
      pend = false;
    }
    // tiles jt + 1 and jt + 2 of the stream go into the other two slots
    if (ahead == 0 && issue_next(std::integral_constant<int, S1>{})) ahead = 1;
    if (ahead == 1 && issue_next(std::integral_constant<int, S2>{})) ahead = 2;
    if (needed) scores(sK[S], sc);
    if (needed) finish(kbase, masked, sV[S], sc);
    if (++jt == C.ntiles) {
      // item end: N's Q fragments (the old ones are dead), then C's output
      if (hasN) {
        wait_vmcnt_atmost<G>(loads - qN);
        read_q();
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): the fragments are read
        asm volatile("" ::: "memory");
      }
      stage();
      if (!hasN) {
        flush(C);
        done = true;
        return;
      }
      P = C;
      pend = true;
      C = N;
      curN = false;
      enter(C);
      jt = 0;
      hasN = advance(rN, N);
    }
    // the next tile has landed (this wave's part of it), then all waves meet
    wait_vmcnt_atmost<G>(loads - e[S1]);
    ring_barrier();
    --ahead;
  };
  using Slot0 = std::integral_constant<int, 0>;
  using Slot1 = std::integral_constant<int, 1>;
  using Slot2 = std::integral_constant<int, 2>;
  for (;;) {
    step(Slot0{});
    if (done) break;
    step(Slot1{});
    if (done) break;
    step(Slot2{});
    if (done) break;
  }
}

// ---------------------------------------------------------------------------
// fp32 kernel: exact fp32 arithmetic.  A block takes QB queries (64, or 16
// when 64-query blocks would leave most compute units idle); each query's
// head dims are split over TPQ = DH / 8 lanes (8 dims per lane), so the
// per-key dot products are short and independent (reduced over the TPQ lanes
// with DPP)
// ---------------------------------------------------------------------------
constexpr int kF32Keys = 32;
constexpr int kF32Dims = 8;    // head dims per lane

template <int DH, int QB>
__global__ __launch_bounds__(QB * (DH / kF32Dims)) void attn_f32_kernel(const AttnArgs a) {
  constexpr int TPQ = DH / kF32Dims;
  constexpr int NT = QB * TPQ;
  constexpr int LPT = kF32Keys * DH / (4 * NT);   // float4 loads of K (and of V) per lane and tile
  static_assert(LPT >= 1 && LPT * 4 * NT == kF32Keys * DH, "whole float4 loads per tile");
  __shared__ __attribute__((aligned(16))) float sK[kF32Keys][DH];
  __shared__ __attribute__((aligned(16))) float sV[kF32Keys][DH];
  __shared__ float sS[kF32Keys][QB];   // each query's scores of the current tile

  int b, h, qtile;
  if (!attn_block(a, blockIdx.x, b, h, qtile)) return;
  const int tid = threadIdx.x;
  const int qi = tid / TPQ;
  const int d0 = (tid - qi * TPQ) * kF32Dims;   // this lane's first head dim
  const int T = a.T, H = a.H, W = a.W;
  const int D = a.heads.dil[h];
  const int64_t rowC = (int64_t)H * DH;
  const int P0 = a.p0;
  const int t0 = qtile * QB;
  const int t_last = min(t0 + QB, T) - 1;
  const int tq = t0 + qi;                 // query row; absolute position P0 + tq
  const bool q_live = tq < T;
  const int tqa = P0 + tq;

  float q[kF32Dims], acc[kF32Dims];
  {
    const float* qp = static_cast<const float*>(a.q) + ((int64_t)b * T + tq) * rowC + h * DH + d0;
#pragma unroll
    for (int i = 0; i < kF32Dims; i += 4) {
      float4 w = q_live ? *reinterpret_cast<const float4*>(qp + i) : make_float4(0.f, 0.f, 0.f, 0.f);
      q[i] = w.x; q[i + 1] = w.y; q[i + 2] = w.z; q[i + 3] = w.w;
    }
#pragma unroll
    for (int i = 0; i < kF32Dims; ++i) acc[i] = 0.f;
  }
  const int ng_hi = n_grid(P0 + t_last, W, D);
  const int ng_me = q_live ? n_grid(tqa, W, D) : 0;
  const int ntile_g = (ng_hi + kF32Keys - 1) / kF32Keys;
  const int j_lo = W > 0 ? max(a.base, P0 + t0 - W + 1) : 0;   // absolute
  const int ntile_w = W > 0 ? (P0 + t_last - j_lo + kF32Keys) / kF32Keys : 0;
  const int win_lo_me = max(0, tqa - W + 1);
  const float* gk = static_cast<const float*>(a.grid_k) + grid_row_offset(a.heads, a.B, b, h, 0, DH);
  const float* gv = static_cast<const float*>(a.grid_v) + ((int64_t)a.B * a.vgoff[h] + (int64_t)b * a.vgcap[h]) * DH;
  const float* ak = W > 0 ? static_cast<const float*>(a.all_k) + (int64_t)b * a.arows * rowC + h * DH : nullptr;
  const float* av = W > 0 ? static_cast<const float*>(a.all_v) + (int64_t)b * a.arows * rowC + h * DH : nullptr;

  // LPT float4 of K and of V per lane and tile (rows r + u * NT * 4 / DH,
  // dims c..c+3); the next tile's are loaded while the current one is
  // computed
  const int r = tid * 4 / DH;
  const int c = tid * 4 - r * DH;
  constexpr int RSTEP = NT * 4 / DH;   // rows between a lane's loads
  const int ntile = ntile_g + ntile_w;
  // first key row of tile `it`: grid row, or all-state buffer row (absolute
  // position - base) for a window tile; nvalid = rows of the tile in use
  auto tile_rows = [&](int it, int& row0, int& nvalid) {
    if (it < ntile_g) {
      row0 = it * kF32Keys; nvalid = ng_hi - row0;
    } else {
      row0 = j_lo + (it - ntile_g) * kF32Keys - a.base;
      nvalid = P0 + t_last + 1 - (row0 + a.base);
    }
  };
  auto fetch = [&](int it, float4* kw, float4* vw) {
    int row0, nvalid;
    tile_rows(it, row0, nvalid);
    const bool g = it < ntile_g;
#pragma unroll
    for (int u = 0; u < LPT; ++u) {
      const int rr = r + u * RSTEP;
      kw[u] = make_float4(0.f, 0.f, 0.f, 0.f);
      vw[u] = kw[u];
      if (rr < nvalid) {
        const int64_t off = (int64_t)(row0 + rr) * (g ? (int64_t)DH : rowC) + c;
        kw[u] = *reinterpret_cast<const float4*>((g ? gk : ak) + off);
        vw[u] = *reinterpret_cast<const float4*>((g ? gv : av) + off);
      }
    }
  };
  float4 kw[LPT], vw[LPT];
  if (ntile > 0) fetch(0, kw, vw);

  float m_run = -INFINITY, l_run = 0.f;
  for (int it = 0; it < ntile; ++it) {
    const bool is_grid = it < ntile_g;
    int row0, nvalid;
    tile_rows(it, row0, nvalid);
    __syncthreads();
#pragma unroll
    for (int u = 0; u < LPT; ++u) {
      *reinterpret_cast<float4*>(&sK[r + u * RSTEP][c]) = kw[u];
      *reinterpret_cast<float4*>(&sV[r + u * RSTEP][c]) = vw[u];
    }
    __syncthreads();
    if (it + 1 < ntile) fetch(it + 1, kw, vw);
    // the tile's scores first (masked keys -inf), then one rescale of the
    // running sums per tile and one exponential per key
    float tmax = -INFINITY;
#pragma unroll 4
    for (int kk = 0; kk < kF32Keys; ++kk) {
      bool valid;
      if (is_grid) {
        valid = row0 + kk < ng_me;
      } else {
        const int j = row0 + a.base + kk;   // absolute position of the key
        valid = j >= win_lo_me && j <= tqa && kk < nvalid;
      }
      float sp = 0.f;
#pragma unroll
      for (int i = 0; i < kF32Dims; ++i) sp = fmaf(q[i], sK[kk][d0 + i], sp);
      sp = group_sum<TPQ>(sp);   // DPP within the query's TPQ adjacent lanes
      const float sc = valid ? sp * a.sl2 : -INFINITY;   // uniform across the lanes of one query
      sS[kk][qi] = sc;   // every lane of a query stores the same value
      tmax = fmaxf(tmax, sc);
    }
    if (tmax > -INFINITY) {
      const float m_new = fmaxf(m_run, tmax);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);   // 0 while m_run is -inf
      l_run *= alpha;
#pragma unroll
      for (int i = 0; i < kF32Dims; ++i) acc[i] *= alpha;
#pragma unroll 4
      for (int kk = 0; kk < kF32Keys; ++kk) {
        const float p = __builtin_amdgcn_exp2f(sS[kk][qi] - m_new);   // 0 for a masked key
        l_run += p;
#pragma unroll
        for (int i = 0; i < kF32Dims; ++i) acc[i] = fmaf(p, sV[kk][d0 + i], acc[i]);
      }
      m_run = m_new;
    }
  }
  if (q_live) {
    const float inv = l_run > 0.f ? 1.0f / l_run : 0.f;
    float* op = static_cast<float*>(a.out) + ((int64_t)b * T + tq) * rowC + h * DH + d0;
#pragma unroll
    for (int i = 0; i < kF32Dims; i += 4)
      *reinterpret_cast<float4*>(op + i) = make_float4(acc[i] * inv, acc[i + 1] * inv, acc[i + 2] * inv, acc[i + 3] * inv);
  }
}

// Dilation classes of the launch (heads sorted by dilation, at most kMaxCls
// classes: the last one takes every remaining head); returns the grid size.
int set_classes(const AttnPlan& p, AttnArgs& a) {
  int idx[kMaxHeads];
  for (int h = 0; h < p.H; ++h) idx[h] = h;
  std::stable_sort(idx, idx + p.H, [&](int x, int y) { return p.heads.dil[x] < p.heads.dil[y]; });
  a.ncls = 0;
  for (int i = 0; i < p.H; ++i) {
    a.hord[i] = (uint8_t)idx[i];
    if (i == 0 || (p.heads.dil[idx[i]] != p.heads.dil[idx[i - 1]] && a.ncls < kMaxCls))
      a.cls_h0[a.ncls++] = i;
  }
  a.cls_h0[a.ncls] = p.H;
  a.cls_b0[0] = 0;
  for (int c = 0; c < a.ncls; ++c) {
    const int n = p.B * (a.cls_h0[c + 1] - a.cls_h0[c]) * a.n_qtiles;
    a.cls_b0[c + 1] = a.cls_b0[c] + (c + 1 < a.ncls ? (n + 7) / 8 * 8 : n);
  }
  return a.cls_b0[a.ncls];
}

}  // namespace

hipError_t launch_prefill_attention(const AttnPlan& p, hipStream_t s) {
  if (p.T <= 0 || p.B <= 0) return hipSuccess;
  if (p.bf16) {
    // 32-bit per-lane byte offsets into the transposed value rows
    const int64_t lim = (int64_t(1) << 31) / p.Dh;
    bool ok = p.tpad <= lim;
    for (int h = 0; h < p.H; ++h) ok = ok && p.vgcap[h] <= lim;
    if (!ok) return hipErrorInvalidValue;
  }
  AttnArgs a;
  a.q = p.q; a.out = p.out;
  a.grid_k = p.grid_k; a.grid_v = p.grid_v;
  a.all_k = p.all_k; a.all_v = p.all_v;
  a.B = p.B; a.T = p.T; a.H = p.H; a.W = p.W;
  a.tpad = p.tpad;
  a.p0 = (int)p.p0;
  a.base = (int)p.base;
  a.arows = p.arows > 0 ? p.arows : p.T;
  a.sl2 = p.scale * 1.4426950408889634f;
  a.heads = p.heads;
  a.sel = p.sel;
  a.sel_k = p.sel_k;
  for (int h = 0; h < kMaxHeads; ++h) {
    a.vgoff[h] = p.vgoff[h];
    a.vgcap[h] = p.vgcap[h];
  }
  if (p.bf16) {
    a.n_qtiles = (p.T + kBM - 1) / kBM;
    const int blocks = set_classes(p, a);
    if (!p.sel && p.W == 0) {
      // persistent blocks, one per compute unit, a multiple of 8 (one per XCD
      // slot), at most one per 8 items
      int dev = 0, cus = 0;
      if (hipGetDevice(&dev) != hipSuccess ||
          hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return hipErrorInvalidDevice;
      const int per_xcd = std::max(1, std::min(cus / 8, (blocks + 7) / 8));
      if (p.Dh == 128)
        hipLaunchKernelGGL((attn_bf16_stream_kernel<128>), dim3(8 * per_xcd), dim3(kWaves * 64), 0, s, a);
      else
        hipLaunchKernelGGL((attn_bf16_stream_kernel<64>), dim3(8 * per_xcd), dim3(kWaves * 64), 0, s, a);
    } else if (p.sel) {
      if (p.Dh == 128)
        hipLaunchKernelGGL((attn_bf16_kernel<128, true>), dim3(blocks), dim3(kWaves * 64), 0, s, a);
      else
        hipLaunchKernelGGL((attn_bf16_kernel<64, true>), dim3(blocks), dim3(kWaves * 64), 0, s, a);
    } else if (p.Dh == 128) {
      hipLaunchKernelGGL((attn_bf16_kernel<128, false>), dim3(blocks), dim3(kWaves * 64), 0, s, a);
    } else {
      hipLaunchKernelGGL((attn_bf16_kernel<64, false>), dim3(blocks), dim3(kWaves * 64), 0, s, a);
    }
  } else {
    // 64-query blocks unless that leaves fewer blocks than compute units
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return hipErrorInvalidDevice;
    const bool small = (int64_t)p.B * p.H * ((p.T + 63) / 64) < cus;
    a.n_qtiles = small ? (p.T + 15) / 16 : (p.T + 63) / 64;
    const int blocks = set_classes(p, a);
    if (small) {
      if (p.Dh == 128)
        hipLaunchKernelGGL((attn_f32_kernel<128, 16>), dim3(blocks), dim3(16 * (128 / kF32Dims)), 0, s, a);
      else
        hipLaunchKernelGGL((attn_f32_kernel<64, 16>), dim3(blocks), dim3(16 * (64 / kF32Dims)), 0, s, a);
    } else if (p.Dh == 128) {
      hipLaunchKernelGGL((attn_f32_kernel<128, 64>), dim3(blocks), dim3(64 * (128 / kF32Dims)), 0, s, a);
    } else {
      hipLaunchKernelGGL((attn_f32_kernel<64, 64>), dim3(blocks), dim3(64 * (64 / kF32Dims)), 0, s, a);
    }
  }
  return hipGetLastError();
}

}  // namespace rat
