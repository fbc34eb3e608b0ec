// k_verify.hip -- checking a draft tree: the packed ancestry mask that lets
// the target verify the whole tree in one forward (PCTree article, "straight
// draft"), and the greedy acceptance walk (DSpark explainer, "one inference,
// from guess to confirmation": keep the run of matches from the root, stop at
// the first mismatch, where the target supplies its own token).
#include "pct_device.h"
#include "pct_internal.h"

namespace pct {

// the first step of the sampling generator, on the host
static uint64_t splitmix64_host(uint64_t x) {
  x += 0x9E3779B97F4A7C15ull;
  x = (x ^ (x >> 30)) * 0xBF58476D1CE4E5B9ull;
  x = (x ^ (x >> 27)) * 0x94D049BB133111EBull;
  return x ^ (x >> 31);
}

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
  int32_t* ts = par + N;
  uint8_t* ok = reinterpret_cast<uint8_t*>(ts + N);
  const int q = blockIdx.x, lane = threadIdx.x;
  const int n = min(n_nodes[q], N);
  const int32_t* T = tok + (int64_t)q * N;
  const int32_t* Pa = parent + (int64_t)q * N;
  const int32_t* D = depth + (int64_t)q * N;
  const int32_t* tg = target + (int64_t)q * (N + 1);
  // match bits, one word per 64 nodes (a whole wave per word); the loads of
  // kAccW words are in flight together (parents and tokens, then the
  // target tokens after the parents)
  constexpr int kAccW = 8;
  for (int w0 = 0; w0 < words; w0 += kAccW) {
    int p[kAccW], tk[kAccW], tt[kAccW];
#pragma unroll
    for (int u = 0; u < kAccW; ++u) {
      const int i = 64 * (w0 + u) + lane;
      const bool in = w0 + u < words && i < n;
      p[u] = in ? Pa[i] : -2;
      tk[u] = in ? T[i] : 0;
    }
#pragma unroll
    for (int u = 0; u < kAccW; ++u) {
      const int i = 64 * (w0 + u) + lane;
      tt[u] = (p[u] >= -1 && p[u] < i) ? tg[p[u] + 1] : 0;
    }
#pragma unroll
    for (int u = 0; u < kAccW; ++u) {
      if (w0 + u >= words) break;
      const int i = 64 * (w0 + u) + lane;
      bool m = false;
      if (i < n) {
        m = (p[u] >= -1 && p[u] < i) && tk[u] == tt[u];
        par[i] = p[u];
        ts[i] = tk[u];
        ok[i] = m;
      }
      const uint64_t b = __ballot(m);
      if (lane == 0) mbits[w0 + u] = b;
    }
  }
  __syncthreads();
  // deepest accepted node: key = depth * 2^20 + (2^20 - 1 - i)
  int best = -1;
  for (int i = lane; i < n; i += kWave) {
    bool acc = true;
    if (mask != nullptr && words <= kAccW) {
      // the node's whole mask row in flight at once
      const uint64_t* row = mask + ((int64_t)q * N + i) * words;
      uint64_t r[kAccW];
#pragma unroll
      for (int w = 0; w < kAccW; ++w) r[w] = w < words ? row[w] : 0;
#pragma unroll
      for (int w = 0; w < kAccW; ++w)
        acc = acc && (w >= words || (r[w] & ~mbits[w]) == 0);
      acc = acc && ok[i];
    } else if (mask != nullptr) {
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
          at[j] = ts[a];
        }
        a = par[a];
      }
      if (dl <= B) at[dl] = tg[leaf + 1];
      tau[q] = dl + 1;
    }
  }
}

// ---------------------------------------------------------------------
// Sampled target tokens (verification with temperature sampling instead of
// greedy decoding): row i of a request's target logits is the target's
// distribution after node i-1 (row 0: after the root), and its token is
// the Gumbel-max sample argmax_v (z_v / T - log(-log(u_v))), ties to the
// lowest token.  u_v is SplitMix64 (Steele, Lea and Flood, 2014) of
// (seed, stream = request * (N+1) + row, v): ((h >> 11) + 0.5) * 2^-53
// with h = sm(sm(sm(seed) ^ stream) ^ v).  Keys are formed in double.
// One workgroup per (row, request); rows past a request's nodes get -1.
__device__ __forceinline__ uint64_t splitmix64(uint64_t x) {
  x += 0x9E3779B97F4A7C15ull;
  x = (x ^ (x >> 30)) * 0xBF58476D1CE4E5B9ull;
  x = (x ^ (x >> 27)) * 0x94D049BB133111EBull;
  return x ^ (x >> 31);
}

constexpr int kSampleThreads = 256;
constexpr int kSampleBlocks = 2048;    // workgroups a call aims for
constexpr int kSampleMinChunk = 2048;  // logits per workgroup at least

struct SamplePart {
  double key;
  int32_t tok;
  int32_t pad;
};

// Arg-max by (key desc, token asc) over the threads of one workgroup; the
// result is valid in thread 0.
__device__ __forceinline__ void block_argmax(double& best, int& bv,
                                             double* wkey, int* wtok,
                                             int tid) {
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const double ok = __shfl_xor(best, d, kWave);
    const int ov = __shfl_xor(bv, d, kWave);
    if (ok > best || (ok == best && ov < bv)) {
      best = ok;
      bv = ov;
    }
  }
  const int lane = tid & 63, wave = tid >> 6;
  if (lane == 0) {
    wkey[wave] = best;
    wtok[wave] = bv;
  }
  __syncthreads();
  if (tid == 0) {
    for (int w = 1; w < kSampleThreads / kWave; ++w)
      if (wkey[w] > best || (wkey[w] == best && wtok[w] < bv)) {
        best = wkey[w];
        bv = wtok[w];
      }
  }
}

// Gumbel-max keys of one slice of one row (grid: slices x rows x
// requests).  With one slice the workgroup writes the sampled token;
// otherwise its (key, token) best goes to part[row][slice] for the merge.
// A row whose keys are all -inf samples token 0 (the first one).
__global__ __launch_bounds__(kSampleThreads) void sample_kernel(
    int N1, int V, int S, int chunk, const float* logits, double inv_t,
    uint64_t seed_mix, const int32_t* n_nodes, int32_t* sampled,
    SamplePart* part) {
  __shared__ double wkey[kSampleThreads / kWave];
  __shared__ int wtok[kSampleThreads / kWave];
  const int c = blockIdx.x, i = blockIdx.y, q = blockIdx.z,
            tid = threadIdx.x;
  const int64_t row = (int64_t)q * N1 + i;
  if (i > n_nodes[q]) {
    if (S == 1 && tid == 0) sampled[row] = -1;
    return;
  }
  const uint64_t key1 = splitmix64(seed_mix ^ (uint64_t)row);
  const float* z = logits + row * V;
  const int v1 = min((c + 1) * chunk, V);
  double best = -__builtin_inf();
  int bv = 0x7fffffff;
  for (int v = c * chunk + tid; v < v1; v += kSampleThreads) {
    const uint64_t h = splitmix64(key1 ^ (uint64_t)v);
    const double u = ((double)(h >> 11) + 0.5) * (1.0 / 9007199254740992.0);
    const double key = (double)z[v] * inv_t + (-log(-log(u)));
    if (key > best) {  // tokens only grow within a thread
      best = key;
      bv = v;
    }
  }
  block_argmax(best, bv, wkey, wtok, tid);
  if (tid == 0) {
    if (S == 1)
      sampled[row] = bv == 0x7fffffff ? 0 : bv;
    else
      part[row * S + c] = SamplePart{best, bv, 0};
  }
}

// One wave per row: the arg-max of the row's S slice results.
__global__ __launch_bounds__(256) void sample_merge_kernel(
    int64_t rows, int N1, int S, const int32_t* n_nodes,
    const SamplePart* part, int32_t* sampled) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int q = (int)(row / N1), i = (int)(row % N1);
  if (i > n_nodes[q]) {
    if (lane == 0) sampled[row] = -1;
    return;
  }
  double best = -__builtin_inf();
  int bv = 0x7fffffff;
  for (int j = lane; j < S; j += kWave) {
    const SamplePart p = part[row * S + j];
    if (p.key > best || (p.key == best && p.tok < bv)) {
      best = p.key;
      bv = p.tok;
    }
  }
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const double ok = __shfl_xor(best, d, kWave);
    const int ov = __shfl_xor(bv, d, kWave);
    if (ok > best || (ok == best && ov < bv)) {
      best = ok;
      bv = ov;
    }
  }
  if (lane == 0) sampled[row] = bv == 0x7fffffff ? 0 : bv;
}

int sample_slices(int64_t rows, int V) {
  int64_t s = (kSampleBlocks + rows - 1) / rows;
  const int64_t smax = V / kSampleMinChunk;
  if (s > smax) s = smax;
  return s < 1 ? 1 : (int)s;
}

size_t sample_workspace(int64_t rows, int V) {
  const int S = sample_slices(rows, V);
  return S > 1 ? (size_t)rows * S * sizeof(SamplePart) : 0;
}

hipError_t launch_sample(int batch, int N1, int V, const float* logits,
                         double inv_t, uint64_t seed, const int32_t* n_nodes,
                         int32_t* sampled, void* ws, hipStream_t s) {
  const int64_t rows = (int64_t)batch * N1;
  const int S = sample_slices(rows, V);
  const int chunk = (V + S - 1) / S;
  SamplePart* part = static_cast<SamplePart*>(ws);
  hipLaunchKernelGGL(sample_kernel, dim3(S, N1, batch), dim3(kSampleThreads),
                     0, s, N1, V, S, chunk, logits, inv_t,
                     splitmix64_host(seed), n_nodes, sampled, part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || S == 1) return e;
  hipLaunchKernelGGL(sample_merge_kernel, dim3((unsigned)((rows + 3) / 4)),
                     dim3(256), 0, s, rows, N1, S, n_nodes, part, sampled);
  return hipGetLastError();
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
  const size_t lds = (size_t)(N + 63) / 64 * 8 + (size_t)N * 9;
  hipError_t e = allow_lds(reinterpret_cast<const void*>(accept_kernel), lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(accept_kernel, dim3(batch), dim3(64), lds, s, N, B, tok,
                     parent, depth, n_nodes, mask, target, tau, accept_node,
                     accept_tok);
  return hipGetLastError();
}

}  // namespace pct
