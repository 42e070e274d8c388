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

// One thread per (b, h, d, r): all-state row r < n_pre (absolute position
// base + r) of channel d takes ring slot (base + r) % W if the position is
// at or after ring_lo (the oldest position the ring still holds), else 0.
template <typename ET>
__global__ void ring_prefix_kernel(const RingPrefixPlan p) {
  const int64_t total = (int64_t)p.B * p.H * p.n_pre * p.Dh;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
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

// One thread per (b, h, d, r) for the rows r of positions ring_from + r:
// ring slot (ring_from + r) % W <- all-state row ring_from - base + r.
template <typename ET>
__global__ void states_to_ring_kernel(const RingPrefixPlan p, int64_t ring_from, int64_t n) {
  const int64_t total = (int64_t)p.B * p.H * n * p.Dh;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
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

// One thread per (b, h, d, column i < vgcap[h]): column i of row d of the
// transposed grid values is grid entry i (zero past rows[h]).  Consecutive
// threads take consecutive columns, so the writes are contiguous.
__global__ void grid_to_col_kernel(const GridColPlan p, int64_t total_cols) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  // locate (h, b, d, col) from the flat index over heads in order
  int64_t rem = i;
  int h = 0;
  for (; h < p.H; ++h) {
    const int64_t n = (int64_t)p.B * p.Dh * p.vgcap[h];
    if (rem < n) break;
    rem -= n;
  }
  if (h >= p.H || i >= total_cols) return;
  const int cap = p.vgcap[h];
  const int col = int(rem % cap);
  rem /= cap;
  const int d = int(rem % p.Dh);
  const int b = int(rem / p.Dh);
  bf16_t v = 0;
  if (col < p.rows[h])
    v = static_cast<const bf16_t*>(p.src)[grid_row_offset(p.heads, p.B, b, h, col, p.Dh) + d];
  static_cast<bf16_t*>(p.dst)[((int64_t)p.B * p.vgoff[h] + (int64_t)b * cap) * p.Dh + (int64_t)d * cap +
                              col_key_pos(col, d)] = v;
}

}  // namespace

hipError_t launch_ring_prefix(const RingPrefixPlan& p, hipStream_t s) {
  const int64_t total = (int64_t)p.B * p.H * p.n_pre * p.Dh;
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
  int64_t total = 0;
  for (int h = 0; h < p.H; ++h) total += (int64_t)p.B * p.Dh * p.vgcap[h];
  if (total <= 0) return hipSuccess;
  const int threads = 256;
  const int64_t blocks = (total + threads - 1) / threads;
  hipLaunchKernelGGL(grid_to_col_kernel, dim3((unsigned)blocks), dim3(threads), 0, s, p, total);
  return hipGetLastError();
}

}  // namespace rat
