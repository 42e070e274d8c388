// Internal declarations shared by the HIP kernels and the C-ABI host layer of
// librat.  gfx950 (CDNA4) only: wave64, bf16 MFMA, hardware bf16 conversion.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rat {

constexpr int kMaxHeads = 128;
constexpr int kMaxCls = 8;   // dilation classes the attention launch orders its blocks by

// ---------------------------------------------------------------------------
// bf16 helpers (storage is raw uint16_t; arithmetic is fp32)
// ---------------------------------------------------------------------------
typedef uint16_t bf16_t;
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));
typedef float floatx16_t __attribute__((ext_vector_type(16)));

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(bf16_t h) { return __uint_as_float(uint32_t(h) << 16); }

// Round-to-nearest-even fp32 -> bf16 (one v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ float round_bf16(float x) {
  return bf16_lo(pack_bf16x2(x, 0.f) & 0xffffu);
}

// ---------------------------------------------------------------------------
// gate: (g, 1-g) = (sigmoid(z), sigmoid(-z)) without cancellation.
// With e = exp(-|z|) in (0, 1]: sigmoid(|z|) = 1/(1+e), sigmoid(-|z|) = e/(1+e).
// z = +inf gives (1, 0), z = -inf gives (0, 1); NaN propagates.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void gate_pair(float z, float& g, float& c) {
  const float e = __builtin_amdgcn_exp2f(-1.4426950408889634f * fabsf(z));
  const float big = __builtin_amdgcn_rcpf(1.0f + e);
  const float small = e * big;
  const bool pos = z >= 0.0f;
  g = pos ? big : small;
  c = pos ? small : big;
}
// sigmoid(-z) = 1 - g by itself, the input weight of the recurrence, as
// 1 / (1 + e^z) (e^z overflowing to inf gives 0, z = -inf gives exactly 1,
// NaN propagates).  Its relative error is that of e^z taken as
// 2^(z log2 e): about |z| ulps from rounding the exponent, a few ulps where
// the value matters.  The prefill scan keeps only this value per element and
// applies the decay as h - c h, with no rounded 1 - c.
__device__ __forceinline__ float gate_comp(float z) {
  return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(1.4426950408889634f * z));
}

// ---------------------------------------------------------------------------
// Per-head tables, passed by value as kernel arguments.
// grid rows of head h live at element offset B*goff[h]*Dh, laid out
// [B][gcap[h]][Dh].
// ---------------------------------------------------------------------------
struct HeadTable {
  int32_t dil[kMaxHeads];
  int32_t gcap[kMaxHeads];
  int64_t goff[kMaxHeads];
};

// Element offset of grid row i of (b, h).
__device__ __forceinline__ int64_t grid_row_offset(const HeadTable& ht, int B, int b, int h,
                                                   int64_t i, int Dh) {
  return ((int64_t)B * ht.goff[h] + (int64_t)b * ht.gcap[h] + i) * Dh;
}

// Workspace header (first 256 bytes of every workspace).
struct WsHeader {
  uint32_t reserved;
  uint32_t epoch;       // scan: call counter; tags published carries
  uint32_t error;       // sticky bit set: a device-side check failed (see rat.h)
  uint32_t poll_limit;  // caller-set: 0 = default look-back polls, n > 0 = n - 1 polls
  uint32_t pad[60];
};
static_assert(sizeof(WsHeader) == 256, "header size");

constexpr uint32_t kErrDecodePos = 2u;    // decode position outside [0, max_pos)

// ---------------------------------------------------------------------------
// Transposed ("column") state layouts used between the scan and the bf16
// attention kernel: per (b, h) a [Dh][cap] matrix, keys along a row, cap a
// multiple of 64.  Inside each 64-key tile of row d the keys sit in eight
// 16-byte chunks: logical chunk c = 2 * (j/16 % 4) + (j/4 % 2) holds keys
// 16s + 4g + {0..3} then 16s + 8 + 4g + {0..3} (s = c/2, g = c%2), which is
// the bf16 operand one MFMA lane needs for a 16-key step, and it is stored
// at physical chunk c ^ col_swz(d).  With 128-byte rows, the 16 lanes that
// read chunk c of 16 consecutive rows hit distinct banks both for a 32-bank
// LDS (8 lanes per cycle) and a 64-bank LDS (16 lanes per cycle).
// ---------------------------------------------------------------------------
__host__ __device__ __forceinline__ int col_swz(int d) { return (d ^ (d >> 3)) & 7; }
__host__ __device__ __forceinline__ int col_chunk(int64_t j) { return int(((j >> 3) & 6) | ((j >> 2) & 1)); }
__host__ __device__ __forceinline__ int64_t col_key_pos(int64_t j, int d) {
  return (j & ~int64_t(63)) | ((col_chunk(j) ^ col_swz(d)) << 3) | (((j >> 3) & 1) << 2) | (j & 3);
}

// ---------------------------------------------------------------------------
// Launchers (host side, defined in the .hip files)
// ---------------------------------------------------------------------------
enum GridMode {
  kGridToken = 0,    // [B][T/D][H][Dh], uniform D (public rat_scan layout)
  kGridHeadRow = 1,  // head h at B*goff[h]*Dh: [B][gcap[h]][Dh]
  kGridHeadCol = 2   // head h at B*goff[h]*Dh: [B][Dh][gcap[h]], col_key_pos order
};
enum AllMode {
  kAllToken = 0,     // [B][T][H][Dh]
  kAllHeadCol = 1    // [B][H][Dh][tpad], col_key_pos order, zero past T
};

struct ScanTensor {
  const void* x;       // [B][T][H][Dh] (f32 or bf16)
  const float* z;      // [B][T][H][Dh]
  const float* h0;     // [B][H][Dh] or null
  void* out_all;       // all states (input dtype) or null
  void* out_grid;      // grid states (input dtype) or null
  float* h_last;       // [B][H][Dh] or null
  int all_mode;        // AllMode of out_all
  int grid_mode;       // GridMode of out_grid
};

// Positions.  Row t of the inputs is absolute position p0 + t: grid entries
// are the states at absolute positions j with (j + 1) % D == 0 (entry
// (j + 1) / D - 1), and all-state outputs put row t at row (or column)
// all_row0 + t of a buffer with arows rows.
struct ScanPlan {
  ScanTensor ten[2];
  int ntensors;
  int B, T, H, Dh;
  int64_t tpad;        // row length of kAllHeadCol (multiple of 64, >= all_row0 + T)
  int64_t p0;          // absolute position of row 0
  int64_t all_row0;    // all-state row of input row 0 (multiple of 64 for kAllHeadCol)
  int64_t arows;       // rows of a kAllToken buffer (>= all_row0 + T)
  int reset_every;     // > 0: chunk-local recurrence, restarted from zero at multiples of it
  int bf16;            // 1: x and outputs are bf16; 0: fp32
  HeadTable heads;
  void* ws;            // workspace base (header + look-back arrays)
  // Optional (null: unused): per tensor, room for one (A, B) fp32 pair per
  // grid element, in the row-major order of the grid (kGridHeadRow or
  // kGridToken indexing; kGridHeadCol grids index it as kGridHeadRow).  With
  // it, a scan that stores only grid states (no all-state output, no restart,
  // every stored D >= 16) runs as a segmented scan.
  float* part[2];
};

// Smallest dilation of a grid-only scan that runs segmented (at most one grid
// position in each wave's steps).
constexpr int kSegMinD = 16;

// Whether a scan plan stores grid states only, with D >= kSegMinD wherever a
// grid is stored: the segmented scan then applies, given part[].
bool scan_grid_only(const ScanPlan& p);
size_t scan_workspace_bytes(int ntensors, int B, int T, int H, int Dh);
hipError_t launch_scan(const ScanPlan& p, hipStream_t s);

// Query row t is absolute position p0 + t; all-state row (or column) r is
// absolute position base + r (base a multiple of 64).  Grid keys use the
// head table `heads`; the grid values, `vgoff` / `vgcap` (element offset
// B * vgoff[h] * Dh, capacity vgcap[h], a multiple of 64 in kGridHeadCol).
struct AttnPlan {
  const void* q;       // [B][T][H][Dh]
  void* out;           // [B][T][H][Dh]
  const void* grid_k;  // grid states, kGridHeadRow
  const void* grid_v;  // bf16: kGridHeadCol; fp32: kGridHeadRow
  const void* all_k;   // all states, kAllToken with arows rows (needed when W > 0)
  const void* all_v;   // bf16: kAllHeadCol; fp32: kAllToken
  int B, T, H, Dh, W;
  int64_t tpad;
  int64_t p0, base, arows;
  int bf16;
  float scale;
  HeadTable heads;
  int64_t vgoff[kMaxHeads];
  int32_t vgcap[kMaxHeads];
  // Block-selection mode (top-k prefill, bf16 only): null for the dilated key
  // set.  Otherwise the key set of a query is block 0, its own 64-position
  // block (causal) and the blocks listed for it in sel [B][T][H][sel_k]
  // (ascending, -1 padded); heads use D = 1 and W = 0, grid_k is the dense
  // key cache and grid_v the values in kAllHeadCol layout with tpad columns.
  const int32_t* sel;
  int sel_k;
};
// Largest top-k of the block-selection mode (its per-query lists sit in LDS).
constexpr int kSelMaxK = 16;
hipError_t launch_prefill_attention(const AttnPlan& p, hipStream_t s);

// Chunked prefill helpers.
// Rows [0, n_pre) of the all-state buffers (absolute positions base + r):
// ring slot (base + r) % W where base + r >= ring_lo, zeros elsewhere.  K in
// kAllToken with arows rows; V in kAllHeadCol (bf16) or kAllToken (fp32).
struct RingPrefixPlan {
  void* ring_k = nullptr; void* ring_v = nullptr;   // [B][H][W][Dh]
  void* all_k = nullptr; void* all_v = nullptr;
  int B = 0, H = 0, Dh = 0, W = 0;
  int64_t base = 0, n_pre = 0, ring_lo = 0, arows = 0, tpad = 0;
  int bf16 = 0;
  // launch_ring_prefix only: fp32 [B][H][Dh] states copied st_* -> h0_* in
  // the same launch (n_state = B * H * Dh elements each; 0: none)
  const float* st_k = nullptr; const float* st_v = nullptr;
  float* h0_k = nullptr; float* h0_v = nullptr;
  int64_t n_state = 0;
};
hipError_t launch_ring_prefix(const RingPrefixPlan& p, hipStream_t s);
// The reverse: ring slots of positions [ring_from, base + arows) from the
// all-state buffers (rows ring_from - base ..).
hipError_t launch_states_to_ring(const RingPrefixPlan& p, int64_t ring_from, hipStream_t s);

// Grid rows [0, rows[h]) of every (b, h) from the row-major cache layout
// (heads.goff / heads.gcap) into the column layout (vgoff / vgcap, zero past
// rows[h] up to vgcap[h]); bf16 only.
struct GridColPlan {
  const void* src; void* dst;
  int B, H, Dh;
  HeadTable heads;
  int64_t vgoff[kMaxHeads];
  int32_t vgcap[kMaxHeads];
  int32_t rows[kMaxHeads];
  // optional, bf16: the ring update of launch_states_to_ring (positions
  // ring_from .. ring_from + ring_n - 1) in the same launch (ring_n 0: none)
  RingPrefixPlan ring;
  int64_t ring_from, ring_n;
};
hipError_t launch_grid_to_col(const GridColPlan& p, hipStream_t s);

struct DecodeHeads {
  HeadTable t;                   // dilation, grid capacity and grid offset by head
  int32_t nsplit[kMaxHeads];     // splits of one (b, h) item, by head
  int32_t order[kMaxHeads];      // heads in launch order (heaviest first)
  int32_t item_base[kMaxHeads + 1];  // first item of order[i]
};

struct DecodePlan {
  const void* q; const void* k; const void* v;   // [B][H][Dh]
  const float* zk; const float* zv;              // [B][H][Dh]
  float* state_k; float* state_v;                // [B][H][Dh]
  void* grid_k; void* grid_v;                    // ragged head-major
  void* ring_k; void* ring_v;                    // [B][H][W][Dh]
  const int32_t* pos;                            // [B]
  int64_t max_pos;
  void* out;                                     // [B][H][Dh]
  int B, H, Dh, W;
  int bf16;
  float scale;
  DecodeHeads heads;
  int n_items;
  int any_split;
  float* partials;                               // [B*H*maxsplit][Dh+2]
  int max_split;
  uint32_t* hdr;
  int reset_every;                               // > 0: state restarts from zero at multiples of it
};
hipError_t launch_decode(const DecodePlan& p, hipStream_t s);

// Top-k block attention over a cache of every recurrent state.  The state
// caches are [H][B][max_pos][Dh] (the grid layout with dilation 1), the
// block summaries fp32 [H][B][max_pos / block][3][Dh] (min, max, mean of the
// key states of each complete block).
constexpr int kTopkMaxBlocks = 8192;   // max_pos / block
constexpr int kTopkMaxK = 128;
enum TopkScore { kTopkQuest = 0, kTopkMoba = 1 };

struct TopkPlan {
  const void* q;        // prefill: [B][T][H][Dh]; decode: [B][H][Dh]
  void* out;            // same layout as q
  int32_t* chosen;      // [.. query ..][topk] or null
  const void* cache_k; const void* cache_v;
  float* summary;
  const int32_t* pos;   // decode: device [B]; prefill: null (query row i is position p0 + i)
  int64_t p0, max_pos;
  int B, T, H, Dh, block, topk, score;
  int bf16;
  float scale;
  uint32_t* hdr;        // decode: workspace header (error word)
  int select_only;      // prefill: write chosen, skip the attention
};
// Summaries of the blocks j in [j_lo, j_hi) of every (h, b).
hipError_t launch_topk_stats(const TopkPlan& p, int64_t j_lo, int64_t j_hi, hipStream_t s);
// Queries (prefill rows or one decode token per sequence): selection and attention.
hipError_t launch_topk_attend(const TopkPlan& p, hipStream_t s);
// Prefill selection only (chosen lists), tiles of 64 queries sharing their
// candidates: bf16, block 64, p0 = 0, T <= kTopkTileMaxT.
constexpr int kTopkTileMaxT = 64 * 257;
hipError_t launch_topk_select_tile(const TopkPlan& p, hipStream_t s);

struct TopkAppendPlan {
  const void* k; const void* v;      // [B][H][Dh]
  const float* zk; const float* zv;
  float* state_k; float* state_v;    // [B][H][Dh]
  void* cache_k; void* cache_v;
  float* summary;
  const int32_t* pos;
  int64_t max_pos;
  int B, H, Dh, block;
  int bf16;
  uint32_t* hdr;
};
// Decode: state update, cache row at pos[b], summary of a block it completes.
hipError_t launch_topk_append(const TopkAppendPlan& p, hipStream_t s);

}  // namespace rat
