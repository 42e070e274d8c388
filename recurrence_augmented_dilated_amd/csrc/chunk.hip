// Helpers of the chunked prefill: continuing a prefill from a decode cache.
//
// A prefill chunk covers absolute positions p0 .. p0+T-1 of sequences whose
// earlier positions live in a decode cache (recurrent state, grid entries,
// window ring).  Its queries need, besides the chunk's own states, the
// window states of the W-1 positions before p0 (from the ring) and every
// grid entry before them (from the cache's grid); the key sets are those of
// "RAT+: Train Dense, Infer Sparse" (abstract and Fig. 1c: every D-th state
// plus an optional local window), with the grid at absolute positions.
#include "rat_internal.h"

namespace rat {
namespace {

// The first 2 n_state threads copy the carried states (keys, then values);
// then one thread per (b, h, d, r): all-state row r < n_pre (absolute
// position base + r) of channel d takes ring slot (base + r) % W if the
// position is at or after ring_lo (the oldest position the ring still
// holds), else 0.
template <typename ET>
__global__ void ring_prefix_kernel(const RingPrefixPlan p) {
  const int64_t total = (int64_t)p.B * p.H * p.n_pre * p.Dh;
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < 2 * p.n_state) {
    if (i < p.n_state) p.h0_k[i] = p.st_k[i];
    else p.h0_v[i - p.n_state] = p.st_v[i - p.n_state];
    return;
  }
  i -= 2 * p.n_state;
  if (i >= total) return;
  const int d = int(i % p.Dh);
  int64_t rest = i / p.Dh;
  const int64_t r = rest % p.n_pre;
  rest /= p.n_pre;
  const int h = int(rest % p.H);
  const int b = int(rest / p.H);
  const int64_t j = p.base + r;
  ET kv = ET(0), vv = ET(0);
  if (j >= p.ring_lo) {
    const int64_t src = (((int64_t)b * p.H + h) * p.W + j % p.W) * p.Dh + d;
    kv = static_cast<const ET*>(p.ring_k)[src];
    vv = static_cast<const ET*>(p.ring_v)[src];
  }
  const int64_t C = (int64_t)p.H * p.Dh;
  static_cast<ET*>(p.all_k)[((int64_t)b * p.arows + r) * C + (int64_t)h * p.Dh + d] = kv;
  if (p.bf16) {
    static_cast<ET*>(p.all_v)[(((int64_t)b * p.H + h) * p.Dh + d) * p.tpad + col_key_pos(r, d)] = vv;
  } else {
    static_cast<ET*>(p.all_v)[((int64_t)b * p.arows + r) * C + (int64_t)h * p.Dh + d] = vv;
  }
}

// One element (b, h, d, r), i = ((b * H + h) * n + r) * Dh + d, of the rows
// r of positions ring_from + r: ring slot (ring_from + r) % W <- all-state
// row ring_from - base + r.
template <typename ET>
__device__ __forceinline__ void ring_update_elem(const RingPrefixPlan& p, int64_t ring_from, int64_t n, int64_t i) {
  const int64_t total = (int64_t)p.B * p.H * n * p.Dh;
  if (i >= total) return;
  const int d = int(i % p.Dh);
  int64_t rest = i / p.Dh;
  const int64_t r = rest % n;
  rest /= n;
  const int h = int(rest % p.H);
  const int b = int(rest / p.H);
  const int64_t j = ring_from + r;            // absolute position
  const int64_t row = j - p.base;             // all-state row
  const int64_t C = (int64_t)p.H * p.Dh;
  const ET kv = static_cast<const ET*>(p.all_k)[((int64_t)b * p.arows + row) * C + (int64_t)h * p.Dh + d];
  const ET vv = p.bf16 ? static_cast<const ET*>(p.all_v)[(((int64_t)b * p.H + h) * p.Dh + d) * p.tpad +
                                                         col_key_pos(row, d)]
                       : static_cast<const ET*>(p.all_v)[((int64_t)b * p.arows + row) * C + (int64_t)h * p.Dh + d];
  const int64_t dst = (((int64_t)b * p.H + h) * p.W + j % p.W) * p.Dh + d;
  static_cast<ET*>(p.ring_k)[dst] = kv;
  static_cast<ET*>(p.ring_v)[dst] = vv;
}

template <typename ET>
__global__ void states_to_ring_kernel(const RingPrefixPlan p, int64_t ring_from, int64_t n) {
  ring_update_elem<ET>(p, ring_from, n, (int64_t)blockIdx.x * blockDim.x + threadIdx.x);
}

// One workgroup per (h, b, 64-entry block of the grid): the block's rows
// (16-byte loads) into a padded LDS tile, then each thread writes whole
// 16-byte chunks of the transposed rows: physical chunk p of row d holds
// logical chunk c = p ^ col_swz(d), i.e. entries 16 (c / 2) + 4 (c % 2) +
// {0..3} and the four 8 further on (col_key_pos order).  Entries at or past
// rows[h] are written as zeros (the attention reads whole 64-key tiles).
template <int DH>
__global__ __launch_bounds__(256) void grid_to_col_kernel(const GridColPlan p) {
  // padded LDS row (bytes, an odd number of dwords): the eight entries a
  // thread gathers and those of the other lanes fall in distinct banks
  constexpr int kRow = DH * 2 + 20;
  __shared__ __attribute__((aligned(16))) char s_t[64 * kRow];
  // locate (h, b, block) from the flat workgroup index over heads in order
  int64_t rem = blockIdx.x;
  int h = 0;
  for (; h < p.H; ++h) {
    const int64_t n = (int64_t)p.B * (p.vgcap[h] / 64);
    if (rem < n) break;
    rem -= n;
  }
  if (h >= p.H) {   // past the grid: the ring update folded into this launch
    if (p.ring_n > 0) ring_update_elem<bf16_t>(p.ring, p.ring_from, p.ring_n, rem * 256 + threadIdx.x);
    return;
  }
  const int nblk = p.vgcap[h] / 64;
  const int b = int(rem / nblk);
  const int jb = int(rem - (int64_t)b * nblk);
  const int tid = threadIdx.x;
  const int rows = p.rows[h];
  const bf16_t* src = static_cast<const bf16_t*>(p.src) + grid_row_offset(p.heads, p.B, b, h, (int64_t)jb * 64, DH);
  constexpr int CPR = DH / 8;   // 16-byte chunks per grid row
#pragma unroll
  for (int k = 0; k < 64 * CPR / 256; ++k) {
    const int e = tid + 256 * k;
    const int r = e / CPR, q = e - r * CPR;
    uint4 w = make_uint4(0, 0, 0, 0);
    if (jb * 64 + r < rows) w = *reinterpret_cast<const uint4*>(src + (int64_t)r * DH + 8 * q);
    uint32_t* t = reinterpret_cast<uint32_t*>(s_t + r * kRow + 16 * q);   // 4-byte aligned only
    t[0] = w.x; t[1] = w.y; t[2] = w.z; t[3] = w.w;
  }
  __syncthreads();
  const int cap = p.vgcap[h];
  bf16_t* dst = static_cast<bf16_t*>(p.dst) + ((int64_t)p.B * p.vgoff[h] + (int64_t)b * cap) * DH + (int64_t)jb * 64;
#pragma unroll
  for (int k = 0; k < DH * 8 / 256; ++k) {
    const int e = tid + 256 * k;
    const int d = e >> 3, ph = e & 7;
    const int c = ph ^ col_swz(d);
    const int j0 = 16 * (c >> 1) + 4 * (c & 1);
    const uint16_t* col = reinterpret_cast<const uint16_t*>(s_t) + d;
    uint32_t v[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[i] = col[(j0 + i) * (kRow / 2)];
      v[4 + i] = col[(j0 + 8 + i) * (kRow / 2)];
    }
    const uint4 w = make_uint4(v[0] | (v[1] << 16), v[2] | (v[3] << 16), v[4] | (v[5] << 16), v[6] | (v[7] << 16));
    *reinterpret_cast<uint4*>(dst + (int64_t)d * cap + 8 * ph) = w;
  }
}

}  // namespace

hipError_t launch_ring_prefix(const RingPrefixPlan& p, hipStream_t s) {
  const int64_t total = (int64_t)p.B * p.H * p.n_pre * p.Dh + 2 * p.n_state;
  if (total <= 0) return hipSuccess;
  const int threads = 256;
  const int64_t blocks = (total + threads - 1) / threads;
  if (p.bf16)
    hipLaunchKernelGGL(ring_prefix_kernel<bf16_t>, dim3((unsigned)blocks), dim3(threads), 0, s, p);
  else
    hipLaunchKernelGGL(ring_prefix_kernel<float>, dim3((unsigned)blocks), dim3(threads), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_states_to_ring(const RingPrefixPlan& p, int64_t ring_from, hipStream_t s) {
  const int64_t n = p.base + p.arows - ring_from;    // positions ring_from .. base + arows - 1
  const int64_t total = (int64_t)p.B * p.H * n * p.Dh;
  if (n <= 0 || total <= 0) return hipSuccess;
  const int threads = 256;
  const int64_t blocks = (total + threads - 1) / threads;
  if (p.bf16)
    hipLaunchKernelGGL(states_to_ring_kernel<bf16_t>, dim3((unsigned)blocks), dim3(threads), 0, s, p, ring_from, n);
  else
    hipLaunchKernelGGL(states_to_ring_kernel<float>, dim3((unsigned)blocks), dim3(threads), 0, s, p, ring_from, n);
  return hipGetLastError();
}

hipError_t launch_grid_to_col(const GridColPlan& p, hipStream_t s) {
  int64_t blocks = 0;
  for (int h = 0; h < p.H; ++h) blocks += (int64_t)p.B * (p.vgcap[h] / 64);
  if (p.ring_n > 0) blocks += ((int64_t)p.B * p.H * p.ring_n * p.Dh + 255) / 256;
  if (blocks <= 0) return hipSuccess;
  if (p.Dh == 128) hipLaunchKernelGGL(grid_to_col_kernel<128>, dim3((unsigned)blocks), dim3(256), 0, s, p);
  else hipLaunchKernelGGL(grid_to_col_kernel<64>, dim3((unsigned)blocks), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace rat
