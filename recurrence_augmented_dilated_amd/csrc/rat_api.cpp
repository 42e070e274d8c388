// C-ABI layer of librat: argument validation (host only, before any HIP
// call), workspace sizing and carving, launch planning.  The operator it
// exposes is documented in include/rat.h.
#include "rat.h"

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "rat_internal.h"

namespace {

thread_local char g_err[512] = "";

rat_status_t fail(rat_status_t st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

rat_status_t ok() {
  g_err[0] = '\0';
  return RAT_OK;
}

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t elt_size(rat_dtype_t dt) { return dt == RAT_BF16 ? 2 : 4; }

rat_status_t check_common(int32_t B, int32_t T, int32_t H, int32_t Dh, rat_dtype_t dt) {
  if (B < 1) return fail(RAT_ERR_INVALID_ARG, "B must be >= 1 (got %d)", B);
  if (T < 0) return fail(RAT_ERR_INVALID_ARG, "T must be >= 0 (got %d)", T);
  if (H < 1 || H > RAT_MAX_HEADS)
    return fail(RAT_ERR_INVALID_ARG, "H must be in [1, %d] (got %d)", RAT_MAX_HEADS, H);
  if (dt != RAT_F32 && dt != RAT_BF16) return fail(RAT_ERR_INVALID_ARG, "unknown dtype %d", (int)dt);
  if (Dh != 64 && Dh != 128) return fail(RAT_ERR_UNSUPPORTED, "Dh must be 64 or 128 (got %d)", Dh);
  return RAT_OK;
}

rat_status_t check_ptr(const void* p, const char* name, bool nullable) {
  if (!p) return nullable ? RAT_OK : fail(RAT_ERR_INVALID_ARG, "%s must not be NULL", name);
  if (!aligned16(p)) return fail(RAT_ERR_INVALID_ARG, "%s must be 16-byte aligned", name);
  return RAT_OK;
}

rat_status_t check_dilation(const int32_t* dilation, int32_t H) {
  if (!dilation) return fail(RAT_ERR_INVALID_ARG, "dilation must not be NULL");
  for (int h = 0; h < H; ++h)
    if (dilation[h] < 1) return fail(RAT_ERR_INVALID_ARG, "dilation[%d] must be >= 1 (got %d)", h, dilation[h]);
  return RAT_OK;
}

// Prefill workspace layout.  Grid states of head h: T / D_h entries per
// sequence; the bf16 path pads every head's capacity to a multiple of 64
// keys (whole attention tiles) and keeps values transposed (kGridHeadCol),
// keys row-major (kGridHeadRow); the fp32 path keeps both row-major.
void prefill_grid_layout(int32_t T, int32_t H, const int32_t* dilation, bool bf16,
                         rat::HeadTable& ht, int64_t& rows) {
  rows = 0;
  std::memset(&ht, 0, sizeof(ht));
  for (int h = 0; h < H; ++h) {
    const int32_t G = T / dilation[h];
    ht.dil[h] = dilation[h];
    ht.gcap[h] = bf16 ? (G + 63) / 64 * 64 : G;
    ht.goff[h] = rows;
    rows += ht.gcap[h];
  }
}

int64_t prefill_tpad(int32_t T) { return ((int64_t)T + 63) / 64 * 64; }

struct PrefillCarve {
  size_t scan_bytes, grid_bytes, allk_bytes, allv_bytes, total;
};

PrefillCarve prefill_carve(int32_t B, int32_t T, int32_t H, int32_t Dh, const int32_t* dilation,
                           int32_t W, rat_dtype_t dt) {
  rat::HeadTable ht;
  int64_t rows;
  const bool bf16 = dt == RAT_BF16;
  prefill_grid_layout(T, H, dilation, bf16, ht, rows);
  PrefillCarve c;
  c.scan_bytes = align_up(rat::scan_workspace_bytes(2, B, T, H, Dh));
  c.grid_bytes = align_up((size_t)B * rows * Dh * elt_size(dt));
  c.allk_bytes = W > 0 ? align_up((size_t)B * T * H * Dh * elt_size(dt)) : 0;
  c.allv_bytes = W > 0 ? align_up((size_t)B * H * Dh * (bf16 ? prefill_tpad(T) : T) * elt_size(dt)) : 0;
  c.total = c.scan_bytes + 2 * c.grid_bytes + c.allk_bytes + c.allv_bytes;
  return c;
}

// Look-back polls before a block recomputes an unpublished predecessor
// itself.  RAT_SCAN_FALLBACK_SPINS overrides the default (tests force 0 to
// exercise the recompute path).
int scan_fallback_spins() {
  const char* e = std::getenv("RAT_SCAN_FALLBACK_SPINS");
  return e ? std::atoi(e) : -1;
}

// Decode split plan: a (b, h) item streams at most ~4096 grid rows per split,
// and small batches are split further so that the launch has >= 2048 items.
constexpr int kMaxSplit = 256;
void decode_splits(int32_t B, int32_t H, const int32_t* dilation, int32_t W, int64_t max_pos,
                   int32_t* nsplit, int32_t& max_split) {
  max_split = 1;
  const int64_t fill = (2048 + (int64_t)B * H - 1) / ((int64_t)B * H);
  for (int h = 0; h < H; ++h) {
    const int64_t rows = max_pos / dilation[h] + 1;
    int64_t want = (rows + 4095) / 4096;
    const int64_t cap_small = (rows + 255) / 256;
    want = std::max<int64_t>(want, std::min<int64_t>(fill, cap_small));
    want = std::min<int64_t>(std::max<int64_t>(want, 1), kMaxSplit);
    nsplit[h] = (int32_t)want;
    max_split = std::max(max_split, nsplit[h]);
  }
  (void)W;
}

}  // namespace

extern "C" {

const char* rat_status_string(rat_status_t s) {
  switch (s) {
    case RAT_OK: return "RAT_OK";
    case RAT_ERR_INVALID_ARG: return "RAT_ERR_INVALID_ARG";
    case RAT_ERR_UNSUPPORTED: return "RAT_ERR_UNSUPPORTED";
    case RAT_ERR_WORKSPACE: return "RAT_ERR_WORKSPACE";
    case RAT_ERR_HIP: return "RAT_ERR_HIP";
  }
  return "RAT_ERR_UNKNOWN";
}

const char* rat_last_error(void) { return g_err; }

// ---------------------------------------------------------------------------
size_t rat_scan_workspace_size(int32_t B, int32_t T, int32_t H, int32_t Dh) {
  if (B < 1 || T < 0 || H < 1 || Dh < 1) return 0;
  return align_up(rat::scan_workspace_bytes(1, B, T, H, Dh));
}

rat_status_t rat_scan(const void* x, const float* z, const float* h0, void* states,
                      int32_t store_every, float* h_last, int32_t B, int32_t T, int32_t H,
                      int32_t Dh, rat_dtype_t dt, void* ws, size_t ws_bytes, hipStream_t stream) {
  rat_status_t st = check_common(B, T, H, Dh, dt);
  if (st != RAT_OK) return st;
  if (store_every < 1) return fail(RAT_ERR_INVALID_ARG, "store_every must be >= 1 (got %d)", store_every);
  if (T == 0) return ok();   // nothing to do; pointers may be NULL
  if ((st = check_ptr(x, "x", false)) != RAT_OK) return st;
  if ((st = check_ptr(z, "z", false)) != RAT_OK) return st;
  if ((st = check_ptr(h0, "h0", true)) != RAT_OK) return st;
  if ((st = check_ptr(states, "states", true)) != RAT_OK) return st;
  if ((st = check_ptr(h_last, "h_last", true)) != RAT_OK) return st;
  if ((st = check_ptr(ws, "ws", false)) != RAT_OK) return st;
  const size_t need = rat_scan_workspace_size(B, T, H, Dh);
  if (ws_bytes < need) return fail(RAT_ERR_WORKSPACE, "workspace %zu < %zu bytes", ws_bytes, need);
  if (T == 0) return ok();

  rat::ScanPlan p;
  std::memset(&p, 0, sizeof(p));
  p.ten[0].x = x;
  p.ten[0].z = z;
  p.ten[0].h0 = h0;
  p.ten[0].out_grid = states;
  p.ten[0].h_last = h_last;
  p.ten[0].grid_mode = rat::kGridToken;
  p.ntensors = 1;
  p.B = B; p.T = T; p.H = H; p.Dh = Dh;
  p.bf16 = dt == RAT_BF16;
  p.heads.dil[0] = store_every;
  p.ws = ws;
  p.fallback_spins = scan_fallback_spins();
  hipError_t e = rat::launch_scan(p, stream);
  if (e != hipSuccess) return fail(RAT_ERR_HIP, "scan launch: %s", hipGetErrorString(e));
  return ok();
}

// ---------------------------------------------------------------------------
size_t rat_dilated_prefill_workspace_size(int32_t B, int32_t T, int32_t H, int32_t Dh,
                                          const int32_t* dilation, int32_t W, rat_dtype_t dt) {
  if (check_common(B, T, H, Dh, dt) != RAT_OK || W < 0 || check_dilation(dilation, H) != RAT_OK)
    return 0;
  return prefill_carve(B, T, H, Dh, dilation, W, dt).total;
}

rat_status_t rat_dilated_prefill(const void* q, const void* k, const void* v, const float* zk,
                                 const float* zv, void* out, int32_t B, int32_t T, int32_t H,
                                 int32_t Dh, const int32_t* dilation, int32_t W, float scale,
                                 rat_dtype_t dt, void* ws, size_t ws_bytes, hipStream_t stream) {
  return rat_dilated_prefill_stage(RAT_STAGE_ALL, q, k, v, zk, zv, out, B, T, H, Dh, dilation, W,
                                   scale, dt, ws, ws_bytes, stream);
}

rat_status_t rat_dilated_prefill_stage(rat_prefill_stage_t stage, const void* q, const void* k,
                                       const void* v, const float* zk, const float* zv, void* out,
                                       int32_t B, int32_t T, int32_t H, int32_t Dh,
                                       const int32_t* dilation, int32_t W, float scale,
                                       rat_dtype_t dt, void* ws, size_t ws_bytes,
                                       hipStream_t stream) {
  if (stage != RAT_STAGE_ALL && stage != RAT_STAGE_RECURRENCE && stage != RAT_STAGE_ATTENTION)
    return fail(RAT_ERR_INVALID_ARG, "unknown stage %d", (int)stage);
  rat_status_t st = check_common(B, T, H, Dh, dt);
  if (st != RAT_OK) return st;
  if (W < 0) return fail(RAT_ERR_INVALID_ARG, "W must be >= 0 (got %d)", W);
  if ((st = check_dilation(dilation, H)) != RAT_OK) return st;
  if (T == 0) return ok();   // nothing to do; pointers may be NULL
  const void* ptrs[] = {q, k, v, zk, zv, out, ws};
  const char* names[] = {"q", "k", "v", "zk", "zv", "out", "ws"};
  for (int i = 0; i < 7; ++i)
    if ((st = check_ptr(ptrs[i], names[i], false)) != RAT_OK) return st;
  const PrefillCarve cv = prefill_carve(B, T, H, Dh, dilation, W, dt);
  if (ws_bytes < cv.total) return fail(RAT_ERR_WORKSPACE, "workspace %zu < %zu bytes", ws_bytes, cv.total);
  if (T == 0) return ok();

  char* base = static_cast<char*>(ws);
  void* grid_k = base + cv.scan_bytes;
  void* grid_v = base + cv.scan_bytes + cv.grid_bytes;
  void* all_k = W > 0 ? base + cv.scan_bytes + 2 * cv.grid_bytes : nullptr;
  void* all_v = W > 0 ? base + cv.scan_bytes + 2 * cv.grid_bytes + cv.allk_bytes : nullptr;
  const bool bf16 = dt == RAT_BF16;

  rat::ScanPlan sp;
  std::memset(&sp, 0, sizeof(sp));
  int64_t rows;
  prefill_grid_layout(T, H, dilation, bf16, sp.heads, rows);
  sp.ten[0] = {k, zk, nullptr, all_k, grid_k, nullptr, rat::kAllToken, rat::kGridHeadRow};
  sp.ten[1] = {v, zv, nullptr, all_v, grid_v, nullptr, bf16 ? rat::kAllHeadCol : rat::kAllToken,
               bf16 ? rat::kGridHeadCol : rat::kGridHeadRow};
  sp.ntensors = 2;
  sp.B = B; sp.T = T; sp.H = H; sp.Dh = Dh;
  sp.tpad = bf16 ? prefill_tpad(T) : T;
  sp.bf16 = bf16;
  sp.ws = ws;
  sp.fallback_spins = scan_fallback_spins();
  if (stage != RAT_STAGE_ATTENTION) {
    hipError_t e = rat::launch_scan(sp, stream);
    if (e != hipSuccess) return fail(RAT_ERR_HIP, "scan launch: %s", hipGetErrorString(e));
  }
  if (stage == RAT_STAGE_RECURRENCE) return ok();

  rat::AttnPlan ap;
  std::memset(&ap, 0, sizeof(ap));
  ap.q = q; ap.out = out;
  ap.grid_k = grid_k; ap.grid_v = grid_v;
  ap.all_k = all_k; ap.all_v = all_v;
  ap.B = B; ap.T = T; ap.H = H; ap.Dh = Dh; ap.W = W;
  ap.tpad = sp.tpad;
  ap.bf16 = dt == RAT_BF16;
  ap.scale = scale > 0.f ? scale : 1.0f / std::sqrt((float)Dh);
  ap.heads = sp.heads;
  hipError_t e = rat::launch_prefill_attention(ap, stream);
  if (e != hipSuccess) return fail(RAT_ERR_HIP, "attention launch: %s", hipGetErrorString(e));
  return ok();
}

// ---------------------------------------------------------------------------
rat_status_t rat_grid_layout(int32_t H, const int32_t* dilation, int64_t max_pos, int64_t* grid_off,
                             int32_t* grid_cap, int64_t* rows) {
  if (H < 1 || H > RAT_MAX_HEADS) return fail(RAT_ERR_INVALID_ARG, "H must be in [1, %d]", RAT_MAX_HEADS);
  rat_status_t st = check_dilation(dilation, H);
  if (st != RAT_OK) return st;
  if (max_pos < 0) return fail(RAT_ERR_INVALID_ARG, "max_pos must be >= 0");
  if (!grid_off || !grid_cap || !rows) return fail(RAT_ERR_INVALID_ARG, "output arrays must not be NULL");
  int64_t acc = 0;
  for (int h = 0; h < H; ++h) {
    const int64_t cap = max_pos / dilation[h];
    if (cap > INT32_MAX) return fail(RAT_ERR_INVALID_ARG, "grid capacity of head %d overflows", h);
    grid_off[h] = acc;
    grid_cap[h] = (int32_t)cap;
    acc += cap;
  }
  *rows = acc;
  return ok();
}

size_t rat_decode_workspace_size(int32_t B, int32_t H, int32_t Dh, const int32_t* dilation, int32_t W,
                                 int64_t max_pos) {
  if (check_common(B, 0, H, Dh, RAT_BF16) != RAT_OK || W < 0 || max_pos < 1 ||
      check_dilation(dilation, H) != RAT_OK)
    return 0;
  int32_t nsplit[RAT_MAX_HEADS];
  int32_t max_split;
  decode_splits(B, H, dilation, W, max_pos, nsplit, max_split);
  return sizeof(rat::WsHeader) + align_up((size_t)B * H * max_split * (Dh + 2) * sizeof(float));
}

rat_status_t rat_decode_step(const void* q, const void* k, const void* v, const float* zk,
                             const float* zv, float* state_k, float* state_v, void* grid_k,
                             void* grid_v, const int64_t* grid_off, const int32_t* grid_cap,
                             void* ring_k, void* ring_v, const int32_t* pos, int64_t max_pos,
                             void* out, int32_t B, int32_t H, int32_t Dh, const int32_t* dilation,
                             int32_t W, float scale, rat_dtype_t dt, void* ws, size_t ws_bytes,
                             hipStream_t stream) {
  rat_status_t st = check_common(B, 0, H, Dh, dt);
  if (st != RAT_OK) return st;
  if (W < 0) return fail(RAT_ERR_INVALID_ARG, "W must be >= 0 (got %d)", W);
  if (max_pos < 1) return fail(RAT_ERR_INVALID_ARG, "max_pos must be >= 1");
  if ((st = check_dilation(dilation, H)) != RAT_OK) return st;
  if (!grid_off || !grid_cap) return fail(RAT_ERR_INVALID_ARG, "grid_off and grid_cap must not be NULL");
  bool any_grid = false;
  for (int h = 0; h < H; ++h) {
    if (grid_off[h] < 0) return fail(RAT_ERR_INVALID_ARG, "grid_off[%d] < 0", h);
    if ((int64_t)grid_cap[h] < max_pos / dilation[h])
      return fail(RAT_ERR_INVALID_ARG, "grid_cap[%d] = %d < max_pos / D = %lld", h, grid_cap[h],
                  (long long)(max_pos / dilation[h]));
    any_grid = any_grid || grid_cap[h] > 0;
  }
  const void* ptrs[] = {q, k, v, zk, zv, state_k, state_v, pos, out, ws};
  const char* names[] = {"q", "k", "v", "zk", "zv", "state_k", "state_v", "pos", "out", "ws"};
  for (int i = 0; i < 10; ++i)
    if ((st = check_ptr(ptrs[i], names[i], false)) != RAT_OK) return st;
  if ((st = check_ptr(grid_k, "grid_k", !any_grid)) != RAT_OK) return st;
  if ((st = check_ptr(grid_v, "grid_v", !any_grid)) != RAT_OK) return st;
  if ((st = check_ptr(ring_k, "ring_k", W == 0)) != RAT_OK) return st;
  if ((st = check_ptr(ring_v, "ring_v", W == 0)) != RAT_OK) return st;
  const size_t need = rat_decode_workspace_size(B, H, Dh, dilation, W, max_pos);
  if (ws_bytes < need) return fail(RAT_ERR_WORKSPACE, "workspace %zu < %zu bytes", ws_bytes, need);

  rat::DecodePlan p;
  std::memset(&p, 0, sizeof(p));
  p.q = q; p.k = k; p.v = v; p.zk = zk; p.zv = zv;
  p.state_k = state_k; p.state_v = state_v;
  p.grid_k = grid_k; p.grid_v = grid_v;
  p.ring_k = ring_k; p.ring_v = ring_v;
  p.pos = pos; p.max_pos = max_pos; p.out = out;
  p.B = B; p.H = H; p.Dh = Dh; p.W = W;
  p.bf16 = dt == RAT_BF16;
  p.scale = scale > 0.f ? scale : 1.0f / std::sqrt((float)Dh);
  int32_t max_split;
  decode_splits(B, H, dilation, W, max_pos, p.heads.nsplit, max_split);
  p.max_split = max_split;
  for (int h = 0; h < H; ++h) {
    p.heads.t.dil[h] = dilation[h];
    p.heads.t.gcap[h] = grid_cap[h];
    p.heads.t.goff[h] = grid_off[h];
    p.heads.order[h] = h;
  }
  // heaviest heads first: most grid rows per sequence, then head index
  std::stable_sort(p.heads.order, p.heads.order + H, [&](int a, int b) {
    return max_pos / dilation[a] > max_pos / dilation[b];
  });
  int64_t items = 0;
  bool any_split = false;
  for (int i = 0; i < H; ++i) {
    p.heads.item_base[i] = (int32_t)items;
    items += (int64_t)B * p.heads.nsplit[p.heads.order[i]];
    any_split = any_split || p.heads.nsplit[p.heads.order[i]] > 1;
  }
  p.heads.item_base[H] = (int32_t)items;
  if (items > INT32_MAX) return fail(RAT_ERR_UNSUPPORTED, "too many work items");
  p.n_items = (int)items;
  p.any_split = any_split;
  p.hdr = reinterpret_cast<uint32_t*>(ws);
  p.partials = reinterpret_cast<float*>(static_cast<char*>(ws) + sizeof(rat::WsHeader));
  hipError_t e = rat::launch_decode(p, stream);
  if (e != hipSuccess) return fail(RAT_ERR_HIP, "decode launch: %s", hipGetErrorString(e));
  return ok();
}

}  // extern "C"
