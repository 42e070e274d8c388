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
#include <mutex>

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

// ---------------------------------------------------------------------------
// Scratch of rat_decode_step_noalloc (its workspace header and split-K
// partials): one fixed array in every GPU's memory, loaded with the library,
// so that the call allocates nothing.  Host code never passes `scratch` to a
// kernel (its name is a host-side stand-in there): the device address comes
// from hipGetSymbolAddress, once per device, with that device current.
// ---------------------------------------------------------------------------
constexpr size_t kNoallocScratchBytes = RAT_DECODE_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The device address of this device's scratch; the stream must belong to
// the current device.
rat_status_t noalloc_scratch(hipStream_t stream, void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(RAT_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(RAT_ERR_UNSUPPORTED, "device %d (at most %d devices)", dev, kMaxDevices);
  if (stream) {
    hipDevice_t sd = -1;
    e = hipStreamGetDevice(stream, &sd);
    if (e != hipSuccess) return fail(RAT_ERR_HIP, "hipStreamGetDevice: %s", hipGetErrorString(e));
    if ((int)sd != dev)
      return fail(RAT_ERR_INVALID_ARG, "the stream belongs to device %d, the current device is %d", (int)sd, dev);
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(RAT_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return RAT_OK;
}

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

// The bf16 attention addresses a transposed value row of `cols` keys with
// 32-bit per-lane byte offsets: cols * Dh * 2 bytes must stay within 2^32.
rat_status_t check_col_span(int64_t cols, int32_t Dh) {
  if (cols * Dh > (int64_t(1) << 31))
    return fail(RAT_ERR_UNSUPPORTED, "bf16 attention over %lld key positions with Dh %d exceeds its limit of 2^31 / Dh",
                (long long)cols, Dh);
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
// With bf16 and a window, a dense head (D = 1) stores no grid: its grid
// entries are the all-state rows, which the attention reads in their place
// (capacity 0 marks such a head).
void prefill_grid_layout(int32_t T, int32_t H, const int32_t* dilation, bool bf16, int32_t W,
                         rat::HeadTable& ht, int64_t& rows) {
  rows = 0;
  std::memset(&ht, 0, sizeof(ht));
  for (int h = 0; h < H; ++h) {
    const int32_t G = T / dilation[h];
    ht.dil[h] = dilation[h];
    ht.gcap[h] = bf16 && W > 0 && dilation[h] == 1 ? 0 : bf16 ? (G + 63) / 64 * 64 : G;
    ht.goff[h] = rows;
    rows += ht.gcap[h];
  }
}

int64_t prefill_tpad(int32_t T) { return ((int64_t)T + 63) / 64 * 64; }

// A prefill without a window whose every head has D >= kSegMinD stores grid
// states only: its scan runs segmented, with an (A, B) pair per grid element
// in the workspace.
bool prefill_segmented(int32_t H, const int32_t* dilation, int32_t W) {
  if (W != 0) return false;
  for (int h = 0; h < H; ++h)
    if (dilation[h] < rat::kSegMinD) return false;
  return true;
}

struct PrefillCarve {
  size_t scan_bytes, grid_bytes, allk_bytes, allv_bytes, part_bytes, total;
};

PrefillCarve prefill_carve(int32_t B, int32_t T, int32_t H, int32_t Dh, const int32_t* dilation,
                           int32_t W, rat_dtype_t dt) {
  rat::HeadTable ht;
  int64_t rows;
  const bool bf16 = dt == RAT_BF16;
  prefill_grid_layout(T, H, dilation, bf16, W, ht, rows);
  PrefillCarve c;
  c.scan_bytes = align_up(rat::scan_workspace_bytes(2, B, T, H, Dh));
  c.grid_bytes = align_up((size_t)B * rows * Dh * elt_size(dt));
  c.allk_bytes = W > 0 ? align_up((size_t)B * T * H * Dh * elt_size(dt)) : 0;
  c.allv_bytes = W > 0 ? align_up((size_t)B * H * Dh * (bf16 ? prefill_tpad(T) : T) * elt_size(dt)) : 0;
  c.part_bytes = prefill_segmented(H, dilation, W) ? align_up((size_t)B * rows * Dh * 2 * sizeof(float)) : 0;
  c.total = c.scan_bytes + 2 * c.grid_bytes + c.allk_bytes + c.allv_bytes + 2 * c.part_bytes;
  return c;
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

// Chunked prefill (positions p0 .. p0+T-1 continuing a decode cache).
// All-state buffers start at absolute position base = max(0, p0 - Wpre),
// Wpre = W - 1 rounded up to 64, so that every window of the chunk's
// queries lies inside them and their tiles stay 64-aligned; rows
// [0, p0 - base) come from the ring.  The bf16 path also keeps the grid
// values every chunk query can see transposed, per head rounded up to 64.
struct ChunkCarve {
  size_t scan_bytes, h0_bytes, allk_bytes, allv_bytes, vcol_bytes, total;
  int64_t base, all_row0, arows, tpad;
  int64_t vgoff[RAT_MAX_HEADS];
  int32_t vgcap[RAT_MAX_HEADS], rows[RAT_MAX_HEADS];
};

int64_t grid_seen(int64_t t_last, int32_t W, int32_t D) {
  const int64_t x = t_last - W + 1;   // grid entries of query t_last: max(0, t-W+1) / D
  return x > 0 ? x / D : 0;
}

ChunkCarve chunk_carve(int32_t B, int32_t T, int32_t H, int32_t Dh, const int32_t* dilation, int32_t W,
                       int64_t p0, rat_dtype_t dt) {
  ChunkCarve c;
  std::memset(&c, 0, sizeof(c));
  const bool bf16 = dt == RAT_BF16;
  const size_t e = elt_size(dt);
  const int64_t wpre = W > 0 ? ((int64_t)W - 1 + 63) / 64 * 64 : 0;
  c.base = std::max<int64_t>(0, p0 - wpre);
  c.all_row0 = p0 - c.base;
  c.arows = c.all_row0 + T;
  c.tpad = (c.arows + 63) / 64 * 64;
  c.scan_bytes = align_up(rat::scan_workspace_bytes(2, B, T, H, Dh));
  c.h0_bytes = align_up((size_t)2 * B * H * Dh * sizeof(float));
  c.allk_bytes = W > 0 ? align_up((size_t)B * c.arows * H * Dh * e) : 0;
  c.allv_bytes = W > 0 ? align_up((size_t)B * H * Dh * (bf16 ? c.tpad : c.arows) * e) : 0;
  int64_t acc = 0;
  for (int h = 0; h < H; ++h) {
    c.rows[h] = (int32_t)grid_seen(p0 + T - 1, W, dilation[h]);
    c.vgcap[h] = bf16 ? (c.rows[h] + 63) / 64 * 64 : 0;
    c.vgoff[h] = acc;
    acc += c.vgcap[h];
  }
  c.vcol_bytes = bf16 ? align_up((size_t)B * acc * Dh * 2) : 0;
  c.total = c.scan_bytes + c.h0_bytes + c.allk_bytes + c.allv_bytes + c.vcol_bytes;
  return c;
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
  if (dt == RAT_BF16 && (st = check_col_span(prefill_tpad(T), Dh)) != RAT_OK) return st;
  const PrefillCarve cv = prefill_carve(B, T, H, Dh, dilation, W, dt);
  if (ws_bytes < cv.total) return fail(RAT_ERR_WORKSPACE, "workspace %zu < %zu bytes", ws_bytes, cv.total);
  if (T == 0) return ok();

  char* base = static_cast<char*>(ws);
  void* grid_k = base + cv.scan_bytes;
  void* grid_v = base + cv.scan_bytes + cv.grid_bytes;
  void* all_k = W > 0 ? base + cv.scan_bytes + 2 * cv.grid_bytes : nullptr;
  void* all_v = W > 0 ? base + cv.scan_bytes + 2 * cv.grid_bytes + cv.allk_bytes : nullptr;
  char* part = base + cv.scan_bytes + 2 * cv.grid_bytes + cv.allk_bytes + cv.allv_bytes;
  const bool bf16 = dt == RAT_BF16;

  rat::ScanPlan sp;
  std::memset(&sp, 0, sizeof(sp));
  int64_t rows;
  prefill_grid_layout(T, H, dilation, bf16, W, sp.heads, rows);
  if (cv.part_bytes) {
    sp.part[0] = reinterpret_cast<float*>(part);
    sp.part[1] = reinterpret_cast<float*>(part + cv.part_bytes);
  }
  sp.ten[0] = {k, zk, nullptr, all_k, grid_k, nullptr, rat::kAllToken, rat::kGridHeadRow};
  sp.ten[1] = {v, zv, nullptr, all_v, grid_v, nullptr, bf16 ? rat::kAllHeadCol : rat::kAllToken,
               bf16 ? rat::kGridHeadCol : rat::kGridHeadRow};
  sp.ntensors = 2;
  sp.B = B; sp.T = T; sp.H = H; sp.Dh = Dh;
  sp.tpad = bf16 ? prefill_tpad(T) : T;
  sp.arows = T;
  sp.bf16 = bf16;
  sp.ws = ws;
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
  ap.arows = T;
  ap.bf16 = dt == RAT_BF16;
  ap.scale = scale > 0.f ? scale : 1.0f / std::sqrt((float)Dh);
  ap.heads = sp.heads;
  for (int h = 0; h < H; ++h) {
    ap.vgoff[h] = sp.heads.goff[h];
    ap.vgcap[h] = sp.heads.gcap[h];
  }
  hipError_t e = rat::launch_prefill_attention(ap, stream);
  if (e != hipSuccess) return fail(RAT_ERR_HIP, "attention launch: %s", hipGetErrorString(e));
  return ok();
}

// ---------------------------------------------------------------------------
size_t rat_prefill_chunk_workspace_size(int32_t B, int32_t T, int32_t H, int32_t Dh,
                                        const int32_t* dilation, int32_t W, int64_t p0,
                                        rat_dtype_t dt) {
  if (check_common(B, T, H, Dh, dt) != RAT_OK || W < 0 || p0 < 0 || check_dilation(dilation, H) != RAT_OK)
    return 0;
  return chunk_carve(B, T, H, Dh, dilation, W, p0, dt).total;
}

static rat_status_t prefill_chunk_impl(const void* q, const void* k, const void* v, const float* zk,
                               const float* zv, void* out, float* state_k, float* state_v,
                               void* grid_k, void* grid_v, const int64_t* grid_off,
                               const int32_t* grid_cap, void* ring_k, void* ring_v, int64_t p0,
                               int64_t max_pos, int32_t B, int32_t T, int32_t H, int32_t Dh,
                               const int32_t* dilation, int32_t W, float scale, rat_dtype_t dt,
                               void* ws, size_t ws_bytes, hipStream_t stream, int32_t reset_every) {
  rat_status_t st = check_common(B, T, H, Dh, dt);
  if (st != RAT_OK) return st;
  if (W < 0) return fail(RAT_ERR_INVALID_ARG, "W must be >= 0 (got %d)", W);
  if ((st = check_dilation(dilation, H)) != RAT_OK) return st;
  if (p0 < 0) return fail(RAT_ERR_INVALID_ARG, "p0 must be >= 0 (got %lld)", (long long)p0);
  if (p0 % 64 != 0) return fail(RAT_ERR_UNSUPPORTED, "p0 must be a multiple of 64 (got %lld)", (long long)p0);
  if (max_pos < 1 || max_pos > INT32_MAX)
    return fail(RAT_ERR_INVALID_ARG, "max_pos must be in [1, 2^31) (got %lld)", (long long)max_pos);
  if (p0 + T > max_pos)
    return fail(RAT_ERR_INVALID_ARG, "p0 + T = %lld exceeds max_pos = %lld", (long long)(p0 + T),
                (long long)max_pos);
  if (!grid_off || !grid_cap) return fail(RAT_ERR_INVALID_ARG, "grid_off and grid_cap must not be NULL");
  bool any_grid = false;
  for (int h = 0; h < H; ++h) {
    if (grid_off[h] < 0) return fail(RAT_ERR_INVALID_ARG, "grid_off[%d] < 0", h);
    if ((int64_t)grid_cap[h] < max_pos / dilation[h])
      return fail(RAT_ERR_INVALID_ARG, "grid_cap[%d] = %d < max_pos / D = %lld", h, grid_cap[h],
                  (long long)(max_pos / dilation[h]));
    any_grid = any_grid || grid_cap[h] > 0;
  }
  if (T == 0) return ok();   // nothing to do; pointers may be NULL
  const void* ptrs[] = {q, k, v, zk, zv, out, state_k, state_v, ws};
  const char* names[] = {"q", "k", "v", "zk", "zv", "out", "state_k", "state_v", "ws"};
  for (int i = 0; i < 9; ++i)
    if ((st = check_ptr(ptrs[i], names[i], false)) != RAT_OK) return st;
  if ((st = check_ptr(grid_k, "grid_k", !any_grid)) != RAT_OK) return st;
  if ((st = check_ptr(grid_v, "grid_v", !any_grid)) != RAT_OK) return st;
  if ((st = check_ptr(ring_k, "ring_k", W == 0)) != RAT_OK) return st;
  if ((st = check_ptr(ring_v, "ring_v", W == 0)) != RAT_OK) return st;
  const ChunkCarve cv = chunk_carve(B, T, H, Dh, dilation, W, p0, dt);
  if (ws_bytes < cv.total) return fail(RAT_ERR_WORKSPACE, "workspace %zu < %zu bytes", ws_bytes, cv.total);

  const bool bf16 = dt == RAT_BF16;
  if (bf16) {
    int64_t span = cv.tpad;
    for (int h = 0; h < H; ++h) span = std::max<int64_t>(span, cv.vgcap[h]);
    if ((st = check_col_span(span, Dh)) != RAT_OK) return st;
  }
  char* wb = static_cast<char*>(ws);
  float* h0k = reinterpret_cast<float*>(wb + cv.scan_bytes);
  float* h0v = h0k + (size_t)B * H * Dh;
  void* all_k = W > 0 ? wb + cv.scan_bytes + cv.h0_bytes : nullptr;
  void* all_v = W > 0 ? wb + cv.scan_bytes + cv.h0_bytes + cv.allk_bytes : nullptr;
  void* vcol = bf16 ? wb + cv.scan_bytes + cv.h0_bytes + cv.allk_bytes + cv.allv_bytes : nullptr;

  rat::HeadTable cache;   // the cache's grid layout
  std::memset(&cache, 0, sizeof(cache));
  for (int h = 0; h < H; ++h) {
    cache.dil[h] = dilation[h];
    cache.gcap[h] = grid_cap[h];
    cache.goff[h] = grid_off[h];
  }

  // 1. the carried states (the scan reads them as h0 from the workspace and
  // writes h_last over state_k / state_v) and 2. the window states before
  // p0, from the ring: one launch
  hipError_t e;
  {
    rat::RingPrefixPlan rp;
    rp.B = B; rp.H = H; rp.Dh = Dh; rp.W = W;
    rp.st_k = state_k; rp.st_v = state_v; rp.h0_k = h0k; rp.h0_v = h0v;
    rp.n_state = (int64_t)B * H * Dh;
    if (W > 0 && cv.all_row0 > 0) {
      rp.ring_k = ring_k; rp.ring_v = ring_v;
      rp.all_k = all_k; rp.all_v = all_v;
      rp.base = cv.base; rp.n_pre = cv.all_row0;
      rp.ring_lo = std::max<int64_t>(0, p0 - W + 1);
      rp.arows = cv.arows; rp.tpad = cv.tpad;
      rp.bf16 = bf16;
    }
    e = rat::launch_ring_prefix(rp, stream);
    if (e != hipSuccess) return fail(RAT_ERR_HIP, "state copy / ring prefix launch: %s", hipGetErrorString(e));
  }

  // 3. the recurrence from the carried states: chunk states, new grid
  //    entries and ring slots into the cache, final states
  rat::ScanPlan sp;
  std::memset(&sp, 0, sizeof(sp));
  sp.ten[0] = {k, zk, h0k, all_k, grid_k, state_k, rat::kAllToken, rat::kGridHeadRow};
  sp.ten[1] = {v, zv, h0v, all_v, grid_v, state_v, bf16 ? rat::kAllHeadCol : rat::kAllToken, rat::kGridHeadRow};
  sp.ntensors = 2;
  sp.B = B; sp.T = T; sp.H = H; sp.Dh = Dh;
  sp.tpad = bf16 ? cv.tpad : cv.arows;
  sp.p0 = p0;
  sp.all_row0 = cv.all_row0;
  sp.arows = cv.arows;
  sp.reset_every = reset_every;
  sp.bf16 = bf16;
  sp.heads = cache;
  sp.ws = ws;
  e = rat::launch_scan(sp, stream);
  if (e != hipSuccess) return fail(RAT_ERR_HIP, "scan launch: %s", hipGetErrorString(e));
  // the chunk's last min(W, T) states into the ring: a launch of its own for
  // fp32, folded into the grid transpose's launch below for bf16
  rat::RingPrefixPlan rr;
  int64_t ring_from = 0, ring_n = 0;
  if (W > 0) {
    rr.ring_k = ring_k; rr.ring_v = ring_v;
    rr.all_k = all_k; rr.all_v = all_v;
    rr.B = B; rr.H = H; rr.Dh = Dh; rr.W = W;
    rr.base = cv.base; rr.n_pre = cv.all_row0;
    rr.ring_lo = 0;
    rr.arows = cv.arows; rr.tpad = cv.tpad;
    rr.bf16 = bf16;
    ring_from = std::max<int64_t>(p0, p0 + T - W);
    ring_n = std::max<int64_t>(0, cv.base + cv.arows - ring_from);
    if (!bf16) {
      e = rat::launch_states_to_ring(rr, ring_from, stream);
      if (e != hipSuccess) return fail(RAT_ERR_HIP, "ring update launch: %s", hipGetErrorString(e));
    }
  }

  // 4. bf16: the grid values the chunk's queries see, transposed
  rat::AttnPlan ap;
  std::memset(&ap, 0, sizeof(ap));
  if (bf16) {
    rat::GridColPlan gp;
    std::memset(&gp, 0, sizeof(gp));
    gp.src = grid_v; gp.dst = vcol;
    gp.B = B; gp.H = H; gp.Dh = Dh;
    gp.heads = cache;
    for (int h = 0; h < H; ++h) {
      gp.vgoff[h] = cv.vgoff[h];
      gp.vgcap[h] = cv.vgcap[h];
      gp.rows[h] = cv.rows[h];
      ap.vgoff[h] = cv.vgoff[h];
      ap.vgcap[h] = cv.vgcap[h];
    }
    gp.ring = rr;
    gp.ring_from = ring_from;
    gp.ring_n = ring_n;
    e = rat::launch_grid_to_col(gp, stream);
    if (e != hipSuccess) return fail(RAT_ERR_HIP, "grid transpose / ring update launch: %s", hipGetErrorString(e));
  } else {
    for (int h = 0; h < H; ++h) {
      ap.vgoff[h] = grid_off[h];
      ap.vgcap[h] = grid_cap[h];
    }
  }

  // 5. attention of the chunk's queries at absolute positions
  ap.q = q; ap.out = out;
  ap.grid_k = grid_k; ap.grid_v = bf16 ? vcol : grid_v;
  ap.all_k = all_k; ap.all_v = all_v;
  ap.B = B; ap.T = T; ap.H = H; ap.Dh = Dh; ap.W = W;
  ap.tpad = bf16 ? cv.tpad : cv.arows;
  ap.p0 = p0; ap.base = cv.base; ap.arows = cv.arows;
  ap.bf16 = bf16;
  ap.scale = scale > 0.f ? scale : 1.0f / std::sqrt((float)Dh);
  ap.heads = cache;
  e = rat::launch_prefill_attention(ap, stream);
  if (e != hipSuccess) return fail(RAT_ERR_HIP, "attention launch: %s", hipGetErrorString(e));
  return ok();
}

rat_status_t rat_prefill_chunk(const void* q, const void* k, const void* v, const float* zk,
                               const float* zv, void* out, float* state_k, float* state_v,
                               void* grid_k, void* grid_v, const int64_t* grid_off,
                               const int32_t* grid_cap, void* ring_k, void* ring_v, int64_t p0,
                               int64_t max_pos, int32_t B, int32_t T, int32_t H, int32_t Dh,
                               const int32_t* dilation, int32_t W, float scale, rat_dtype_t dt,
                               void* ws, size_t ws_bytes, hipStream_t stream) {  return prefill_chunk_impl(q, k, v, zk, zv, out, state_k, state_v, grid_k, grid_v, grid_off, grid_cap, ring_k,
                            ring_v, p0, max_pos, B, T, H, Dh, dilation, W, scale, dt, ws, ws_bytes, stream, 0);
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
  // one (m, l, acc[Dh]) partial per work item (b, h, split)
  size_t items = 0;
  for (int h = 0; h < H; ++h) items += (size_t)B * nsplit[h];
  return sizeof(rat::WsHeader) + align_up(items * (Dh + 2) * sizeof(float));
}

static rat_status_t decode_step_impl(const void* q, const void* k, const void* v, const float* zk,
                             const float* zv, float* state_k, float* state_v, void* grid_k,
                             void* grid_v, const int64_t* grid_off, const int32_t* grid_cap,
                             void* ring_k, void* ring_v, const int32_t* pos, int64_t max_pos,
                             void* out, int32_t B, int32_t H, int32_t Dh, const int32_t* dilation,
                             int32_t W, float scale, rat_dtype_t dt, void* ws, size_t ws_bytes,
                             hipStream_t stream, int32_t reset_every, bool check_only) {
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
  if (check_only) return ok();

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
  p.reset_every = reset_every;
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

rat_status_t rat_decode_step(const void* q, const void* k, const void* v, const float* zk,
                             const float* zv, float* state_k, float* state_v, void* grid_k,
                             void* grid_v, const int64_t* grid_off, const int32_t* grid_cap,
                             void* ring_k, void* ring_v, const int32_t* pos, int64_t max_pos,
                             void* out, int32_t B, int32_t H, int32_t Dh, const int32_t* dilation,
                             int32_t W, float scale, rat_dtype_t dt, void* ws, size_t ws_bytes,
                             hipStream_t stream) {
  return decode_step_impl(q, k, v, zk, zv, state_k, state_v, grid_k, grid_v, grid_off, grid_cap, ring_k, ring_v,
                          pos, max_pos, out, B, H, Dh, dilation, W, scale, dt, ws, ws_bytes, stream, 0, false);
}

rat_status_t rat_decode_step_noalloc(const void* q, const void* k, const void* v, const float* zk,
                                     const float* zv, float* state_k, float* state_v, void* grid_k,
                                     void* grid_v, const int64_t* grid_off, const int32_t* grid_cap,
                                     void* ring_k, void* ring_v, const int32_t* pos, int64_t max_pos,
                                     void* out, int32_t B, int32_t H, int32_t Dh,
                                     const int32_t* dilation, int32_t W, float scale, rat_dtype_t dt,
                                     hipStream_t stream) {
  // every argument is validated on the host first, with the scratch standing
  // in for the workspace (a placeholder address: nothing is launched here)
  rat_status_t st = check_common(B, 0, H, Dh, dt);
  if (st != RAT_OK) return st;
  if (W >= 0 && max_pos >= 1 && check_dilation(dilation, H) == RAT_OK) {
    const size_t need = rat_decode_workspace_size(B, H, Dh, dilation, W, max_pos);
    if (need > kNoallocScratchBytes)
      return fail(RAT_ERR_WORKSPACE,
                  "this step needs %zu bytes of scratch; rat_decode_step_noalloc has %zu "
                  "(use rat_decode_step with a workspace)", need, kNoallocScratchBytes);
  }
  void* const placeholder = reinterpret_cast<void*>(uintptr_t(kAlign));
  st = decode_step_impl(q, k, v, zk, zv, state_k, state_v, grid_k, grid_v, grid_off, grid_cap, ring_k, ring_v,
                        pos, max_pos, out, B, H, Dh, dilation, W, scale, dt, placeholder, kNoallocScratchBytes,
                        stream, 0, true);
  if (st != RAT_OK) return st;
  void* ws = nullptr;
  if ((st = noalloc_scratch(stream, &ws)) != RAT_OK) return st;
  return decode_step_impl(q, k, v, zk, zv, state_k, state_v, grid_k, grid_v, grid_off, grid_cap, ring_k, ring_v,
                          pos, max_pos, out, B, H, Dh, dilation, W, scale, dt, ws, kNoallocScratchBytes, stream, 0,
                          false);
}

}  // extern "C"

// ---------------------------------------------------------------------------
// top-k block attention
// ---------------------------------------------------------------------------
namespace {

rat_status_t check_topk(int32_t block, int32_t topk, rat_topk_score_t score, int64_t max_pos) {
  if (block < 1 || block > 1024) return fail(RAT_ERR_INVALID_ARG, "block must be in [1, 1024] (got %d)", block);
  if (topk < 0 || topk > rat::kTopkMaxK)
    return fail(RAT_ERR_INVALID_ARG, "topk must be in [0, %d] (got %d)", rat::kTopkMaxK, topk);
  if (score != RAT_TOPK_QUEST && score != RAT_TOPK_MOBA)
    return fail(RAT_ERR_INVALID_ARG, "unknown block score %d", (int)score);
  if (max_pos < 1 || max_pos > INT32_MAX)
    return fail(RAT_ERR_INVALID_ARG, "max_pos must be in [1, 2^31) (got %lld)", (long long)max_pos);
  if (max_pos / block > rat::kTopkMaxBlocks)
    return fail(RAT_ERR_UNSUPPORTED, "max_pos / block = %lld exceeds %d blocks", (long long)(max_pos / block),
                rat::kTopkMaxBlocks);
  return RAT_OK;
}

// the scan writes every state into the [H][B][max_pos][Dh] caches: the grid
// layout with dilation 1 and capacity max_pos on every head
void dense_cache_table(int32_t H, int64_t max_pos, rat::HeadTable& ht) {
  std::memset(&ht, 0, sizeof(ht));
  for (int h = 0; h < H; ++h) {
    ht.dil[h] = 1;
    ht.gcap[h] = (int32_t)max_pos;
    ht.goff[h] = (int64_t)h * max_pos;
  }
}

}  // namespace

extern "C" {

size_t rat_topk_prefill_workspace_size(int32_t B, int32_t T, int32_t H, int32_t Dh) {
  if (check_common(B, T, H, Dh, RAT_BF16) != RAT_OK) return 0;
  // scan workspace, h0 copies, and for the bf16 block-selection path the
  // values in kAllHeadCol layout plus the chosen lists
  const int64_t tpad = (T + 63) / 64 * 64;
  return align_up(rat::scan_workspace_bytes(2, B, T, H, Dh)) + align_up((size_t)2 * B * H * Dh * sizeof(float)) +
         align_up((size_t)B * H * Dh * tpad * 2) + align_up((size_t)B * T * H * rat::kSelMaxK * sizeof(int32_t));
}

rat_status_t rat_topk_prefill(const void* q, const void* k, const void* v, const float* zk,
                              const float* zv, void* out, int32_t* chosen, float* state_k,
                              float* state_v, void* cache_k, void* cache_v, float* summary,
                              int64_t p0, int64_t max_pos, int32_t B, int32_t T, int32_t H,
                              int32_t Dh, int32_t block, int32_t topk, rat_topk_score_t score,
                              float scale, rat_dtype_t dt, void* ws, size_t ws_bytes,
                              hipStream_t stream) {
  rat_status_t st = check_common(B, T, H, Dh, dt);
  if (st != RAT_OK) return st;
  if ((st = check_topk(block, topk, score, max_pos)) != RAT_OK) return st;
  if (p0 < 0) return fail(RAT_ERR_INVALID_ARG, "p0 must be >= 0 (got %lld)", (long long)p0);
  if (p0 + T > max_pos)
    return fail(RAT_ERR_INVALID_ARG, "p0 + T = %lld exceeds max_pos = %lld", (long long)(p0 + T),
                (long long)max_pos);
  if (T == 0) return ok();
  const void* ptrs[] = {q, k, v, zk, zv, out, state_k, state_v, cache_k, cache_v, summary, ws};
  const char* names[] = {"q", "k", "v", "zk", "zv", "out", "state_k", "state_v", "cache_k", "cache_v",
                         "summary", "ws"};
  for (int i = 0; i < 12; ++i)
    if ((st = check_ptr(ptrs[i], names[i], false)) != RAT_OK) return st;
  if ((st = check_ptr(chosen, "chosen", true)) != RAT_OK) return st;
  const size_t need = rat_topk_prefill_workspace_size(B, T, H, Dh);
  if (ws_bytes < need) return fail(RAT_ERR_WORKSPACE, "workspace %zu < %zu bytes", ws_bytes, need);

  const bool bf16 = dt == RAT_BF16;
  const size_t scan_bytes = align_up(rat::scan_workspace_bytes(2, B, T, H, Dh));
  float* h0k = reinterpret_cast<float*>(static_cast<char*>(ws) + scan_bytes);
  float* h0v = h0k + (size_t)B * H * Dh;
  const size_t sbytes = (size_t)B * H * Dh * sizeof(float);
  // Block-selection path: a first pass writes every query's chosen blocks,
  // then the MFMA prefill attention runs over the dense cache with the key
  // set block 0 + chosen + own block (64-position blocks = its key tiles).
  // It needs the values transposed (written by the scan alongside the cache)
  // and so starts at position 0; other calls take one workgroup per query
  // (as do sequences past the MFMA kernel's 2^31 / Dh positions).
  const int64_t tpad = (T + 63) / 64 * 64;
  const bool fast = bf16 && block == 64 && topk <= rat::kSelMaxK && p0 == 0 && tpad * Dh <= (int64_t(1) << 31);
  char* vcol = reinterpret_cast<char*>(h0k) + align_up(2 * sbytes);
  int32_t* sel = reinterpret_cast<int32_t*>(vcol + align_up((size_t)B * H * Dh * tpad * 2));
  // the carried states into the workspace (the scan reads h0 there and writes
  // h_last over state_k / state_v), one small launch for both
  rat::RingPrefixPlan cp;
  cp.st_k = state_k; cp.st_v = state_v; cp.h0_k = h0k; cp.h0_v = h0v;
  cp.n_state = (int64_t)B * H * Dh;
  hipError_t e = rat::launch_ring_prefix(cp, stream);
  if (e != hipSuccess) return fail(RAT_ERR_HIP, "state copy: %s", hipGetErrorString(e));

  // recurrence: every state of positions p0 .. p0+T-1 into the caches
  rat::ScanPlan sp;
  std::memset(&sp, 0, sizeof(sp));
  sp.ten[0] = {k, zk, h0k, nullptr, cache_k, state_k, rat::kAllToken, rat::kGridHeadRow};
  sp.ten[1] = {v, zv, h0v, fast ? vcol : nullptr, cache_v, state_v,
               fast ? rat::kAllHeadCol : rat::kAllToken, rat::kGridHeadRow};
  sp.ntensors = 2;
  sp.B = B; sp.T = T; sp.H = H; sp.Dh = Dh;
  sp.tpad = fast ? tpad : T;
  sp.p0 = p0;
  sp.arows = T;
  sp.bf16 = bf16;
  dense_cache_table(H, max_pos, sp.heads);
  sp.ws = ws;
  e = rat::launch_scan(sp, stream);
  if (e != hipSuccess) return fail(RAT_ERR_HIP, "scan launch: %s", hipGetErrorString(e));

  rat::TopkPlan tp;
  std::memset(&tp, 0, sizeof(tp));
  tp.q = q; tp.out = out; tp.chosen = chosen;
  tp.cache_k = cache_k; tp.cache_v = cache_v; tp.summary = summary;
  tp.p0 = p0; tp.max_pos = max_pos;
  tp.B = B; tp.T = T; tp.H = H; tp.Dh = Dh; tp.block = block; tp.topk = topk; tp.score = (int)score;
  tp.bf16 = bf16;
  tp.scale = scale > 0.f ? scale : 1.0f / std::sqrt((float)Dh);
  // summaries of the blocks whose last position falls in this call
  const int64_t j_lo = (p0 + block) / block - 1;        // first j with (j + 1) * block - 1 >= p0
  const int64_t j_hi = (p0 + T) / block;                 // j with (j + 1) * block <= p0 + T
  e = rat::launch_topk_stats(tp, j_lo, j_hi, stream);
  if (e != hipSuccess) return fail(RAT_ERR_HIP, "block summary launch: %s", hipGetErrorString(e));
  if (!fast) {
    e = rat::launch_topk_attend(tp, stream);
    if (e != hipSuccess) return fail(RAT_ERR_HIP, "top-k attention launch: %s", hipGetErrorString(e));
    return ok();
  }
  int32_t* lists = chosen ? chosen : sel;
  tp.chosen = lists;
  tp.select_only = 1;
  e = T <= rat::kTopkTileMaxT ? rat::launch_topk_select_tile(tp, stream) : rat::launch_topk_attend(tp, stream);
  if (e != hipSuccess) return fail(RAT_ERR_HIP, "top-k selection launch: %s", hipGetErrorString(e));
  rat::AttnPlan ap;
  std::memset(&ap, 0, sizeof(ap));
  ap.q = q; ap.out = out;
  ap.grid_k = cache_k; ap.grid_v = vcol;
  ap.B = B; ap.T = T; ap.H = H; ap.Dh = Dh; ap.W = 0;
  ap.tpad = tpad;
  ap.arows = T;
  ap.bf16 = 1;
  ap.scale = tp.scale;
  dense_cache_table(H, max_pos, ap.heads);
  ap.sel = lists;
  ap.sel_k = topk;
  e = rat::launch_prefill_attention(ap, stream);
  if (e != hipSuccess) return fail(RAT_ERR_HIP, "top-k attention launch: %s", hipGetErrorString(e));
  return ok();
}

rat_status_t rat_topk_summarize(const void* cache_k, float* summary, int64_t j_lo, int64_t j_hi,
                                int64_t max_pos, int32_t B, int32_t H, int32_t Dh, int32_t block,
                                rat_dtype_t dt, hipStream_t stream) {
  rat_status_t st = check_common(B, 0, H, Dh, dt);
  if (st != RAT_OK) return st;
  if ((st = check_topk(block, 0, RAT_TOPK_QUEST, max_pos)) != RAT_OK) return st;
  if (j_lo < 0 || j_hi < j_lo || j_hi > max_pos / block)
    return fail(RAT_ERR_INVALID_ARG, "need 0 <= j_lo <= j_hi <= max_pos / block (got %lld, %lld)",
                (long long)j_lo, (long long)j_hi);
  if (j_hi == j_lo) return ok();
  if ((st = check_ptr(cache_k, "cache_k", false)) != RAT_OK) return st;
  if ((st = check_ptr(summary, "summary", false)) != RAT_OK) return st;
  rat::TopkPlan tp;
  std::memset(&tp, 0, sizeof(tp));
  tp.cache_k = cache_k; tp.summary = summary;
  tp.max_pos = max_pos;
  tp.B = B; tp.H = H; tp.Dh = Dh; tp.block = block;
  tp.bf16 = dt == RAT_BF16;
  hipError_t e = rat::launch_topk_stats(tp, j_lo, j_hi, stream);
  if (e != hipSuccess) return fail(RAT_ERR_HIP, "block summary launch: %s", hipGetErrorString(e));
  return ok();
}

size_t rat_topk_decode_workspace_size(void) { return sizeof(rat::WsHeader); }

rat_status_t rat_topk_decode_step(const void* q, const void* k, const void* v, const float* zk,
                                  const float* zv, float* state_k, float* state_v, void* cache_k,
                                  void* cache_v, float* summary, const int32_t* pos,
                                  int64_t max_pos, void* out, int32_t* chosen, int32_t B, int32_t H,
                                  int32_t Dh, int32_t block, int32_t topk, rat_topk_score_t score,
                                  float scale, rat_dtype_t dt, void* ws, size_t ws_bytes,
                                  hipStream_t stream) {
  rat_status_t st = check_common(B, 0, H, Dh, dt);
  if (st != RAT_OK) return st;
  if ((st = check_topk(block, topk, score, max_pos)) != RAT_OK) return st;
  const void* ptrs[] = {q, k, v, zk, zv, state_k, state_v, cache_k, cache_v, summary, pos, out, ws};
  const char* names[] = {"q", "k", "v", "zk", "zv", "state_k", "state_v", "cache_k", "cache_v", "summary",
                         "pos", "out", "ws"};
  for (int i = 0; i < 13; ++i)
    if ((st = check_ptr(ptrs[i], names[i], false)) != RAT_OK) return st;
  if ((st = check_ptr(chosen, "chosen", true)) != RAT_OK) return st;
  if (ws_bytes < rat_topk_decode_workspace_size())
    return fail(RAT_ERR_WORKSPACE, "workspace %zu < %zu bytes", ws_bytes, rat_topk_decode_workspace_size());
  const bool bf16 = dt == RAT_BF16;
  uint32_t* hdr = static_cast<uint32_t*>(ws);

  rat::TopkAppendPlan ap;
  std::memset(&ap, 0, sizeof(ap));
  ap.k = k; ap.v = v; ap.zk = zk; ap.zv = zv;
  ap.state_k = state_k; ap.state_v = state_v;
  ap.cache_k = cache_k; ap.cache_v = cache_v; ap.summary = summary;
  ap.pos = pos; ap.max_pos = max_pos;
  ap.B = B; ap.H = H; ap.Dh = Dh; ap.block = block;
  ap.bf16 = bf16;
  ap.hdr = hdr;
  hipError_t e = rat::launch_topk_append(ap, stream);
  if (e != hipSuccess) return fail(RAT_ERR_HIP, "append launch: %s", hipGetErrorString(e));

  rat::TopkPlan tp;
  std::memset(&tp, 0, sizeof(tp));
  tp.q = q; tp.out = out; tp.chosen = chosen;
  tp.cache_k = cache_k; tp.cache_v = cache_v; tp.summary = summary;
  tp.pos = pos; tp.max_pos = max_pos;
  tp.B = B; tp.T = 1; tp.H = H; tp.Dh = Dh; tp.block = block; tp.topk = topk; tp.score = (int)score;
  tp.bf16 = bf16;
  tp.scale = scale > 0.f ? scale : 1.0f / std::sqrt((float)Dh);
  tp.hdr = hdr;
  e = rat::launch_topk_attend(tp, stream);
  if (e != hipSuccess) return fail(RAT_ERR_HIP, "top-k attention launch: %s", hipGetErrorString(e));
  return ok();
}

// ---------------------------------------------------------------------------
// RAT chunk-local variant: restart every L positions, D = L, W = 1
// ---------------------------------------------------------------------------
static bool local_dilation(int32_t H, int32_t L, int32_t* dil) {
  if (H < 1 || H > RAT_MAX_HEADS || L < 1) return false;
  for (int h = 0; h < H; ++h) dil[h] = L;
  return true;
}

size_t rat_local_prefill_chunk_workspace_size(int32_t B, int32_t T, int32_t H, int32_t Dh, int32_t L,
                                              int64_t p0, rat_dtype_t dt) {
  int32_t dil[RAT_MAX_HEADS];
  if (!local_dilation(H, L, dil)) return 0;
  return rat_prefill_chunk_workspace_size(B, T, H, Dh, dil, 1, p0, dt);
}

rat_status_t rat_local_prefill_chunk(const void* q, const void* k, const void* v, const float* zk,
                                     const float* zv, void* out, float* state_k, float* state_v,
                                     void* grid_k, void* grid_v, const int64_t* grid_off,
                                     const int32_t* grid_cap, void* ring_k, void* ring_v, int64_t p0,
                                     int64_t max_pos, int32_t B, int32_t T, int32_t H, int32_t Dh,
                                     int32_t L, float scale, rat_dtype_t dt, void* ws, size_t ws_bytes,
                                     hipStream_t stream) {
  int32_t dil[RAT_MAX_HEADS];
  if (!local_dilation(H, L, dil))
    return fail(RAT_ERR_INVALID_ARG, "need 1 <= H <= %d and L >= 1 (got H = %d, L = %d)", RAT_MAX_HEADS, H, L);
  return prefill_chunk_impl(q, k, v, zk, zv, out, state_k, state_v, grid_k, grid_v, grid_off, grid_cap, ring_k,
                            ring_v, p0, max_pos, B, T, H, Dh, dil, 1, scale, dt, ws, ws_bytes, stream, L);
}

size_t rat_local_decode_workspace_size(int32_t B, int32_t H, int32_t Dh, int32_t L, int64_t max_pos) {
  int32_t dil[RAT_MAX_HEADS];
  if (!local_dilation(H, L, dil)) return 0;
  return rat_decode_workspace_size(B, H, Dh, dil, 1, max_pos);
}

rat_status_t rat_local_decode_step(const void* q, const void* k, const void* v, const float* zk,
                                   const float* zv, float* state_k, float* state_v, void* grid_k,
                                   void* grid_v, const int64_t* grid_off, const int32_t* grid_cap,
                                   void* ring_k, void* ring_v, const int32_t* pos, int64_t max_pos,
                                   void* out, int32_t B, int32_t H, int32_t Dh, int32_t L, float scale,
                                   rat_dtype_t dt, void* ws, size_t ws_bytes, hipStream_t stream) {
  int32_t dil[RAT_MAX_HEADS];
  if (!local_dilation(H, L, dil))
    return fail(RAT_ERR_INVALID_ARG, "need 1 <= H <= %d and L >= 1 (got H = %d, L = %d)", RAT_MAX_HEADS, H, L);
  return decode_step_impl(q, k, v, zk, zv, state_k, state_v, grid_k, grid_v, grid_off, grid_cap, ring_k, ring_v,
                          pos, max_pos, out, B, H, Dh, dil, 1, scale, dt, ws, ws_bytes, stream, L, false);
}

}  // extern "C"
