// GPU twin of hkv_inputs/gen.py: the same seeded synthetic keys, values and
// queries, bit for bit (Philox4x32-10 words -> Irwin-Hall normal -> fp32 ->
// bf16 round-to-nearest-even; queries in fp64 then fp32 then bf16).  Input
// generation only: none of the HeadKV method's arithmetic lives here.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

struct Ctr { uint32_t x, y, z, w; };

__device__ inline Ctr philox4x32_10(Ctr c, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
    const uint32_t lo0 = 0xD2511F53u * c.x, hi0 = __umulhi(0xD2511F53u, c.x);
    const uint32_t lo1 = 0xCD9E8D57u * c.z, hi1 = __umulhi(0xCD9E8D57u, c.z);
    c = Ctr{hi1 ^ c.y ^ k0, lo1, hi0 ^ c.w ^ k1, lo0};
  }
  return c;
}

__device__ inline uint32_t halves(uint32_t w) { return (w & 0xffffu) + (w >> 16); }

// z * 65536 as an integer: sum of twelve 16-bit uniforms minus 12 * 32767.5,
// returned doubled to stay integral.
__device__ inline int normal2x(uint32_t idx, uint32_t stream, uint32_t tag, uint32_t k0,
                               uint32_t k1) {
  const Ctr a = philox4x32_10(Ctr{idx, stream, tag, 0u}, k0, k1);
  const Ctr b = philox4x32_10(Ctr{idx, stream, tag, 1u}, k0, k1);
  const int tot = int(halves(a.x) + halves(a.y) + halves(a.z) + halves(a.w) + halves(b.x) +
                      halves(b.y));
  return 2 * tot - 12 * 65535;
}

__device__ inline uint16_t f32_to_bf16(float x) {
  uint32_t u = __float_as_uint(x);
  u += 0x7fffu + ((u >> 16) & 1u);
  return uint16_t(u >> 16);
}

__device__ inline float bits_to_f32(const void* base, long long i, int bf16) {
  if (bf16) return __uint_as_float(uint32_t(static_cast<const uint16_t*>(base)[i]) << 16);
  return static_cast<const float*>(base)[i];
}

__device__ inline void store(void* base, long long i, float v, int bf16) {
  if (bf16) static_cast<uint16_t*>(base)[i] = f32_to_bf16(v);
  else static_cast<float*>(base)[i] = v;
}

// out[s, e] for e in [0, n_per_stream): z of (e, s, tag)
__global__ void k_gen_normal(void* out, int bf16, uint32_t k0, uint32_t k1, uint32_t tag,
                             long long S, long long n_per_stream) {
  const long long total = S * n_per_stream;
  for (long long i = blockIdx.x * (long long)blockDim.x + threadIdx.x; i < total;
       i += (long long)gridDim.x * blockDim.x) {
    const long long s = i / n_per_stream;
    const uint32_t e = uint32_t(i - s * n_per_stream);
    const int z2 = normal2x(e, uint32_t(s), tag, k0, k1);
    const float z = float(z2) / 131072.0f;          // exact
    store(out, i, z, bf16);
  }
}

// Q[s, r, c] for positions t = P - W + r, r in [0, q_rows)
__global__ void k_gen_query(void* Q, const void* K, const uint8_t* local, const int* anchors,
                            int full_history, int bf16, uint32_t k0, uint32_t k1, long long S,
                            int N, int P, int W, int d) {
  const int q_rows = N - P + W;
  const long long total = S * q_rows * (long long)d;
  for (long long i = blockIdx.x * (long long)blockDim.x + threadIdx.x; i < total;
       i += (long long)gridDim.x * blockDim.x) {
    const long long s = i / ((long long)q_rows * d);
    const int rem = int(i - s * (long long)q_rows * d);
    const int r = rem / d, c = rem % d;
    const int t = P - W + r;
    const long long krow = s * (long long)N * d;
    double sum = 0.0, m = 0.0;
    if (local[s]) {
      const int lo = t - 3 > 0 ? t - 3 : 0;
      for (int j = lo; j <= t; ++j) sum += double(bits_to_f32(K, krow + (long long)j * d + c, bf16));
      m = double(t + 1 - lo);
    } else {
      for (int a = 0; a < 4; ++a) {
        const int pos = anchors[s * 4 + a];
        if (full_history && pos > t - 32) continue;
        sum += double(bits_to_f32(K, krow + (long long)pos * d + c, bf16));
        m += 1.0;
      }
    }
    const int e2 = normal2x(uint32_t(t * d + c), uint32_t(s), 2u, k0, k1);
    const double eps = double(e2) / 131072.0;
    const double q64 = (2.0 * sum) / m + 0.5 * eps;
    store(Q, i, float(q64), bf16);
  }
}

int grid_for(long long total) {
  long long g = (total + 255) / 256;
  return int(g < 65536 ? g : 65536);
}

}  // namespace

extern "C" {

// Keys (tag 0) or values (tag 1): out [S, N*d] in fp32 (bf16 = 0) or bf16 bits.
int hkvgen_normal(void* out, int bf16, uint32_t seed, uint32_t cid, uint32_t tag, long long S,
                  long long n_per_stream, void* stream) {
  const long long total = S * n_per_stream;
  if (total <= 0) return 0;
  hipLaunchKernelGGL(k_gen_normal, dim3(grid_for(total)), dim3(256), 0,
                     static_cast<hipStream_t>(stream), out, bf16, seed, cid, tag, S,
                     n_per_stream);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

// Queries from the stored keys; local [S] (1 = locality-biased), anchors [S, 4].
int hkvgen_query(void* Q, const void* K, const uint8_t* local, const int* anchors,
                 int full_history, int bf16, uint32_t seed, uint32_t cid, long long S, int N,
                 int P, int W, int d, void* stream) {
  const long long total = S * (long long)(N - P + W) * d;
  if (total <= 0) return 0;
  hipLaunchKernelGGL(k_gen_query, dim3(grid_for(total)), dim3(256), 0,
                     static_cast<hipStream_t>(stream), Q, K, local, anchors, full_history, bf16,
                     seed, cid, S, N, P, W, d);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

}  // extern "C"
