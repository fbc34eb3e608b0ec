// k_verify.hip -- checking a draft tree: the packed ancestry mask that lets
// the target verify the whole tree in one forward (PCTree article, "straight
// draft"), and the greedy acceptance walk (DSpark explainer, "one inference,
// from guess to confirmation": keep the run of matches from the root, stop at
// the first mismatch, where the target supplies its own token).
#include "pct_device.h"
#include "pct_internal.h"

namespace pct {

// One thread per (request, row, 64-bit word).  Ancestors have smaller
// indices than their descendants (nodes are in key order), so the walk up
// from row i can stop as soon as it leaves word w.
__global__ __launch_bounds__(256) void mask_kernel(int batch, int N,
                                                   int words,
                                                   const int32_t* parent,
                                                   const int32_t* n_nodes,
                                                   uint64_t* mask) {
  const int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t total = (int64_t)batch * N * words;
  if (g >= total) return;
  const int w = (int)(g % words);
  const int i = (int)((g / words) % N);
  const int q = (int)(g / ((int64_t)words * N));
  uint64_t bits = 0;
  if (i < n_nodes[q] && (i >> 6) >= w) {
    const int32_t* par = parent + (int64_t)q * N;
    int a = i;
    while (a >= 0 && (a >> 6) >= w) {
      if ((a >> 6) == w) bits |= (uint64_t)1 << (a & 63);
      const int na = par[a];
      if (na >= a) break;  // malformed input: parents must precede children
      a = na;
    }
  }
  mask[g] = bits;
}

// One wave per request.  Node i is accepted when its token equals the
// target's token after its parent and every ancestor is accepted; accepted
// nodes form a single root path (siblings have distinct tokens), whose
// deepest node gives tau = depth + 1.
// With the packed ancestry mask the test is one pass of word operations:
// the nodes whose token matches form a bit set, and node i is accepted
// exactly when its mask row (itself and its ancestors) lies inside that
// set.  Without it, each node follows its parent links instead.
__global__ __launch_bounds__(64) void accept_kernel(
    int N, int B, const int32_t* tok, const int32_t* parent,
    const int32_t* depth, const int32_t* n_nodes, const uint64_t* mask,
    const int32_t* target, int32_t* tau, int32_t* accept_node,
    int32_t* accept_tok) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int words = (N + 63) / 64;
  uint64_t* mbits = reinterpret_cast<uint64_t*>(smem);
  int32_t* par = reinterpret_cast<int32_t*>(mbits + words);
  uint8_t* ok = reinterpret_cast<uint8_t*>(par + N);
  const int q = blockIdx.x, lane = threadIdx.x;
  const int n = min(n_nodes[q], N);
  const int32_t* T = tok + (int64_t)q * N;
  const int32_t* Pa = parent + (int64_t)q * N;
  const int32_t* D = depth + (int64_t)q * N;
  const int32_t* tg = target + (int64_t)q * (N + 1);
  // match bits, one word per 64 nodes (a whole wave per word)
  for (int w = 0; w < words; ++w) {
    const int i = 64 * w + lane;
    bool m = false;
    if (i < n) {
      const int p = Pa[i];
      par[i] = p;
      m = (p >= -1 && p < i) && T[i] == tg[p + 1];
      ok[i] = m;
    }
    const uint64_t b = __ballot(m);
    if (lane == 0) mbits[w] = b;
  }
  __syncthreads();
  // deepest accepted node: key = depth * 2^20 + (2^20 - 1 - i)
  int best = -1;
  for (int i = lane; i < n; i += kWave) {
    bool acc = true;
    if (mask != nullptr) {
      const uint64_t* row = mask + ((int64_t)q * N + i) * words;
      for (int w = 0; w < words && acc; ++w) acc = (row[w] & ~mbits[w]) == 0;
      acc = acc && ok[i];
    } else {
      int a = i, steps = 0;
      while (a >= 0 && steps <= B) {
        if (!ok[a]) {
          acc = false;
          break;
        }
        a = par[a];
        ++steps;
      }
      acc = acc && a < 0;
    }
    if (acc) {
      const int key = D[i] * (1 << 20) + ((1 << 20) - 1 - i);
      best = key > best ? key : best;
    }
  }
  best = wave_max(best);
  if (lane == 0) {
    int32_t* an = accept_node + (int64_t)q * B;
    int32_t* at = accept_tok + (int64_t)q * (B + 1);
    for (int j = 0; j < B; ++j) an[j] = -1;
    for (int j = 0; j <= B; ++j) at[j] = -1;
    if (best < 0) {
      at[0] = tg[0];
      tau[q] = 1;
    } else {
      const int leaf = (1 << 20) - 1 - (best & ((1 << 20) - 1));
      const int dl = best >> 20;
      int a = leaf;
      for (int j = dl - 1; j >= 0 && a >= 0; --j) {
        if (j < B) {
          an[j] = a;
          at[j] = T[a];
        }
        a = par[a];
      }
      if (dl <= B) at[dl] = tg[leaf + 1];
      tau[q] = dl + 1;
    }
  }
}

hipError_t launch_mask(int batch, int N, const int32_t* parent,
                       const int32_t* n_nodes, uint64_t* mask, hipStream_t s) {
  const int words = (N + 63) / 64;
  const int64_t total = (int64_t)batch * N * words;
  const int blocks = (int)((total + 255) / 256);
  hipLaunchKernelGGL(mask_kernel, dim3(blocks), dim3(256), 0, s, batch, N,
                     words, parent, n_nodes, mask);
  return hipGetLastError();
}

hipError_t launch_accept(int batch, int N, int B, const int32_t* tok,
                         const int32_t* parent, const int32_t* depth,
                         const int32_t* n_nodes, const uint64_t* mask,
                         const int32_t* target, int32_t* tau,
                         int32_t* accept_node, int32_t* accept_tok,
                         hipStream_t s) {
  const size_t lds = (size_t)(N + 63) / 64 * 8 + (size_t)N * 5;
  hipLaunchKernelGGL(accept_kernel, dim3(batch), dim3(64), lds, s, N, B, tok,
                     parent, depth, n_nodes, mask, target, tau, accept_node,
                     accept_tok);
  return hipGetLastError();
}

}  // namespace pct
