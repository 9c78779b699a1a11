// Measurement probes for the roofline ceilings the benchmark reports
// (libmsa_calib.so; not part of the attention library).  Each probe is the
// simplest kernel that moves bytes in one pattern as fast as this GPU
// allows, so a kernel's achieved rate can be read against what its own
// access pattern can reach, not only against the 8 TB/s HBM peak:
//
//   calib_read    streaming read of a large buffer (16-byte non-temporal
//                 loads, every workgroup striding through the array; a
//                 checksum per workgroup keeps the loads alive)
//   calib_write   streaming write of a large buffer (16-byte non-temporal
//                 stores)
//   calib_mixed   streaming read and streaming write at once, WPR 4 KiB
//                 blocks written per block read (16-byte non-temporal loads
//                 and stores, each workgroup owning one chunk of each
//                 array): what DRAM gives when both directions share it.
//   calib_gather  gather of 4 KiB units -- two 2 KiB runs 8 KiB apart, the
//                 K and V rows of one 4-token microblock in a K/V-interleaved
//                 cache of 16-token blocks -- named by a list of unit ids
//                 into a pool small enough to stay in the Infinity Cache:
//                 the ceiling of the grouped microblock route's K/V gather.
//                 Each workgroup keeps UPI units (UPI * 4 KiB) in flight.
//   calib_lds     LDS read throughput of the grouped route's operand reads:
//                 each wave reads one 16 KiB quarter of a 64 KiB buffer (two
//                 16-row tiles of 512-byte rows) over and over, as K
//                 fragments (ds_read_b128, lane (n, q) reads row n at chunk
//                 (8 q + c) ^ s(n), with s(n) the 4-bit row index bit-reversed
//                 as the head_dim 256 kernel stores K, or s(n) = n), as
//                 transposed V fragments (ds_read_b64_tr_b16, row 4 q +
//                 (lane / 4) % 4, chunk 2 (j ^ row % 8) + (lane % 4) / 2), or
//                 as consecutive 16-byte reads.  Two workgroups of 4 waves
//                 per CU, as the grouped attention kernel runs.
//   calib_lds_pattern  LDS read throughput of any one read pattern: 16
//                 instructions of 64 lane offsets given by the caller
//                 (ds_read_b128 or ds_read_b64_tr_b16), the same for every
//                 wave, repeated; the offsets are masked into the 64 KiB
//                 buffer.  It measures which XOR swizzle of a K tile keeps the
//                 reads of an MFMA operand apart on the LDS banks.
//
// All indexing is bounded by the sizes passed in; every kernel exits.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;

__device__ __forceinline__ uint32_t wave_xor(uint32_t x) {
  for (int off = 32; off > 0; off >>= 1) x ^= (uint32_t)__shfl_xor((int)x, off);
  return x;
}

__global__ void __launch_bounds__(kThreads) k_read(const u32x4 *__restrict__ src, int64_t n16,
                                                   uint32_t *__restrict__ sink) {
  constexpr int U = 8;  // independent loads in flight per thread
  uint32_t acc = 0;
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  for (; i + (U - 1) * stride < n16; i += U * stride) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  for (; i < n16; i += stride) {
    const u32x4 v = __builtin_nontemporal_load(src + i);
    acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
  // one word per wave, so no load above can be dropped
  acc = wave_xor(acc);
  if ((threadIdx.x & 63) == 0) sink[blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6)] = acc;
}

// The same read with each workgroup owning one contiguous chunk of the
// array, U consecutive 4 KiB blocks per iteration.
__global__ void __launch_bounds__(kThreads) k_read_chunk(const u32x4 *__restrict__ src, int64_t n16,
                                                         uint32_t *__restrict__ sink) {
  constexpr int U = 8;
  const int64_t per = (n16 / gridDim.x) / (U * kThreads) * (U * kThreads);  // whole iterations
  const int64_t lo = (int64_t)blockIdx.x * per;
  uint32_t acc = 0;
  for (int64_t i = lo + threadIdx.x; i < lo + per; i += U * kThreads) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = __builtin_nontemporal_load(src + i + u * kThreads);
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  acc = wave_xor(acc);
  if ((threadIdx.x & 63) == 0) sink[blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6)] = acc;
}

__global__ void __launch_bounds__(kThreads) k_write(u32x4 *__restrict__ dst, int64_t n16, uint32_t seed) {
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n16; i += stride) {
    const uint32_t x = (uint32_t)i ^ seed;
    __builtin_nontemporal_store(u32x4{x, x + 1u, x + 2u, x + 3u}, dst + i);
  }
}

// Write with each workgroup owning one contiguous chunk, U 4 KiB blocks per
// iteration; TEMPORAL selects ordinary (write-back) stores.
template <bool TEMPORAL>
__global__ void __launch_bounds__(kThreads) k_write_chunk(u32x4 *__restrict__ dst, int64_t n16, uint32_t seed) {
  constexpr int U = 4;
  const int64_t per = (n16 / gridDim.x) / (U * kThreads) * (U * kThreads);
  const int64_t lo = (int64_t)blockIdx.x * per;
  for (int64_t i = lo + threadIdx.x; i < lo + per; i += U * kThreads) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t x = (uint32_t)(i + u * kThreads) ^ seed;
      const u32x4 v = u32x4{x, x + 1u, x + 2u, x + 3u};
      if constexpr (TEMPORAL) dst[i + u * kThreads] = v;
      else __builtin_nontemporal_store(v, dst + i + u * kThreads);
    }
  }
}

// Per iteration a workgroup reads 2 blocks of 4 KiB and writes 2 * WPR; it
// owns `iters` iterations of each array (the caller sizes the arrays).
template <int WPR>
__global__ void __launch_bounds__(kThreads) k_mixed(const u32x4 *__restrict__ src, u32x4 *__restrict__ dst,
                                                    int64_t iters, uint32_t *__restrict__ sink) {
  const int64_t lo_r = (int64_t)blockIdx.x * iters * 2 * kThreads;
  const int64_t lo_w = (int64_t)blockIdx.x * iters * 2 * WPR * kThreads;
  uint32_t acc = 0;
  for (int64_t it = 0; it < iters; ++it) {
    const u32x4 v0 = __builtin_nontemporal_load(src + lo_r + it * 2 * kThreads + threadIdx.x);
    const u32x4 v1 = __builtin_nontemporal_load(src + lo_r + it * 2 * kThreads + kThreads + threadIdx.x);
#pragma unroll
    for (int u = 0; u < 2 * WPR; ++u) {
      const uint32_t x = (uint32_t)(it * 2 * WPR + u) ^ threadIdx.x;
      __builtin_nontemporal_store(u32x4{x, x + 1u, x + 2u, x + 3u},
                                  dst + lo_w + (it * 2 * WPR + u) * kThreads + threadIdx.x);
    }
    acc ^= v0[0] ^ v0[1] ^ v0[2] ^ v0[3] ^ v1[0] ^ v1[1] ^ v1[2] ^ v1[3];
  }
  acc = wave_xor(acc);
  if ((threadIdx.x & 63) == 0) sink[blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6)] = acc;
}

// Unit u of the pool: 16-byte chunks [u4 + c] for c < 128 (K half) and
// [u4 + 512 + c] for c < 128 (V half), u4 = (u / 4) * 1024 + (u % 4) * 128
// in 16-byte units -- block b = u / 4 holds 16 K rows then 16 V rows of 512
// bytes each, unit u % 4 covers 4 rows of each.  Thread t of a workgroup
// loads chunk t % 128 of half t / 128 of each of its UPI units.
template <int UPI>
__global__ void __launch_bounds__(kThreads) k_gather(const u32x4 *__restrict__ pool, int64_t pool16,
                                                     const int32_t *__restrict__ units, int64_t n_units,
                                                     uint32_t *__restrict__ sink) {
  const int half = threadIdx.x >> 7, c = threadIdx.x & 127;
  uint32_t acc = 0;
  for (int64_t base = (int64_t)blockIdx.x * UPI; base < n_units; base += (int64_t)gridDim.x * UPI) {
    int64_t off[UPI];
#pragma unroll
    for (int k = 0; k < UPI; ++k) {
      const int64_t j = base + k;
      const int64_t u = j < n_units ? units[j] : -1;
      const int64_t o = (u / 4) * 1024 + (u % 4) * 128 + half * 512 + c;
      off[k] = (u >= 0 && o < pool16) ? o : -1;
    }
    u32x4 v[UPI];
#pragma unroll
    for (int k = 0; k < UPI; ++k) v[k] = off[k] >= 0 ? pool[off[k]] : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int k = 0; k < UPI; ++k) acc ^= v[k][0] ^ v[k][1] ^ v[k][2] ^ v[k][3];
  }
  acc = wave_xor(acc);
  if ((threadIdx.x & 63) == 0) sink[blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6)] = acc;
}

typedef short i16x4 __attribute__((ext_vector_type(4)));
#define LDS_AS __attribute__((address_space(3)))

template <int MODE>
__global__ void __launch_bounds__(kThreads, 2) k_lds(uint32_t *__restrict__ sink, int iters) {
  __shared__ __attribute__((aligned(16))) uint8_t s[65536];
  const int t = threadIdx.x, lane = t & 63, n = lane & 15, q = lane >> 4;
  for (int i = t; i < 65536 / 16; i += kThreads)
    ((u32x4 *)s)[i] = u32x4{(uint32_t)i, (uint32_t)i * 2654435761u, ~(uint32_t)i, (uint32_t)i ^ 0x5bd1e995u};
  __syncthreads();
  uint32_t acc = 0;
  uint32_t base = (uint32_t)(t >> 6) * 16384u;  // this wave's quarter: rows 0..31 of 512 bytes
  const int vr = q * 4 + ((lane >> 2) & 3), vc = lane & 3;
  for (int it = 0; it < iters; ++it) {
    __asm__ volatile("" : "+v"(base));  // the reads are not hoisted out of the loop
#pragma unroll
    for (int tile = 0; tile < 2; ++tile) {
      const uint32_t tb = base + tile * 8192u;
      if constexpr (MODE == 0 || MODE == 3) {
        const int sw = MODE == 0 ? (int)(__builtin_bitreverse32((uint32_t)n) >> 28) : n;
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          const u32x4 v = *(const u32x4 *)(s + tb + n * 512 + (((8 * q + c) ^ sw) << 4));
          acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
        }
      } else if constexpr (MODE == 1) {
#pragma unroll
        for (int mt = 0; mt < 16; ++mt) {
          const uint32_t o = tb + vr * 512 + (((((mt & 7) ^ (vr & 7)) << 1) + (vc >> 1)) << 4) + (vc & 1) * 8 +
                             (mt & 8) * 32;
          const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4 *)(s + o));
          acc ^= (uint32_t)(uint16_t)v[0] ^ ((uint32_t)(uint16_t)v[1] << 16) ^ (uint32_t)(uint16_t)v[2] ^
                 ((uint32_t)(uint16_t)v[3] << 16);
        }
      } else {
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          const u32x4 v = *(const u32x4 *)(s + tb + c * 1024 + lane * 16);
          acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
        }
      }
    }
  }
  sink[(int64_t)blockIdx.x * kThreads + t] = acc;
}

template <int KIND>  // 0: ds_read_b128, 1: ds_read_b64_tr_b16
__global__ void __launch_bounds__(kThreads, 2) k_lds_pattern(uint32_t *__restrict__ sink, int iters,
                                                            const uint32_t *__restrict__ tab) {
  __shared__ __attribute__((aligned(16))) uint8_t s[65536];
  const int t = threadIdx.x, lane = t & 63;
  for (int i = t; i < 65536 / 16; i += kThreads)
    ((u32x4 *)s)[i] = u32x4{(uint32_t)i, (uint32_t)i * 2654435761u, ~(uint32_t)i, (uint32_t)i ^ 0x5bd1e995u};
  uint32_t off[16];
#pragma unroll
  for (int k = 0; k < 16; ++k) off[k] = tab[k * 64 + lane] & (KIND == 0 ? 0xfff0u : 0xfff8u);
  __syncthreads();
  uint32_t acc = 0, z = 0;
  for (int it = 0; it < iters; ++it) {
    __asm__ volatile("" : "+v"(z));  // the reads are not hoisted out of the loop
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      if constexpr (KIND == 0) {
        const u32x4 v = *(const u32x4 *)(s + (off[k] | z));
        acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
      } else {
        const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4 *)(s + (off[k] | z)));
        acc ^= (uint32_t)(uint16_t)v[0] ^ ((uint32_t)(uint16_t)v[1] << 16) ^ (uint32_t)(uint16_t)v[2] ^
               ((uint32_t)(uint16_t)v[3] << 16);
      }
    }
  }
  sink[(int64_t)blockIdx.x * kThreads + t] = acc;
}

}  // namespace

extern "C" {

// LDS pattern probe: tab holds 16 x 64 byte offsets (device memory), sink
// grid * 256 words; kind 0: ds_read_b128 (16 KiB per wave and iteration),
// kind 1: ds_read_b64_tr_b16 (8 KiB).
int calib_lds_pattern(uint32_t *sink, int grid, int iters, const uint32_t *tab, int kind, void *stream) {
  if (!sink || !tab || grid < 1 || iters < 1 || kind < 0 || kind > 1) return 1;
  const hipStream_t s = (hipStream_t)stream;
  if (kind == 0) k_lds_pattern<0><<<grid, kThreads, 0, s>>>(sink, iters, tab);
  else k_lds_pattern<1><<<grid, kThreads, 0, s>>>(sink, iters, tab);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

// LDS probe: sink holds grid * 256 words; each wave reads 16 KiB per
// iteration.  mode 0: K fragments, bit-reversed row swizzle; 1: transposed
// V fragments; 2: consecutive 16-byte reads; 3: K fragments, row-index
// swizzle.
int calib_lds(uint32_t *sink, int grid, int iters, int mode, void *stream) {
  if (!sink || grid < 1 || iters < 1 || mode < 0 || mode > 3) return 1;
  const hipStream_t s = (hipStream_t)stream;
  switch (mode) {
    case 0: k_lds<0><<<grid, kThreads, 0, s>>>(sink, iters); break;
    case 1: k_lds<1><<<grid, kThreads, 0, s>>>(sink, iters); break;
    case 2: k_lds<2><<<grid, kThreads, 0, s>>>(sink, iters); break;
    default: k_lds<3><<<grid, kThreads, 0, s>>>(sink, iters); break;
  }
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

// sink: one uint32 per wave (4 * grid words).  mode 0: grid-stride
// addressing; mode 1: one contiguous chunk per workgroup (the chunked form
// covers the largest multiple of grid * 32 KiB; the caller counts those
// bytes: calib_chunk_bytes).
int calib_read(const void *src, int64_t bytes, uint32_t *sink, int grid, int mode, void *stream) {
  if (!src || !sink || bytes < 16 || grid < 1 || mode < 0 || mode > 1) return 1;
  const hipStream_t s = (hipStream_t)stream;
  if (mode == 0) k_read<<<grid, kThreads, 0, s>>>((const u32x4 *)src, bytes / 16, sink);
  else k_read_chunk<<<grid, kThreads, 0, s>>>((const u32x4 *)src, bytes / 16, sink);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

// mode 0: grid-stride non-temporal; 1: chunked non-temporal; 2: chunked
// write-back.
int calib_write(void *dst, int64_t bytes, int grid, uint32_t seed, int mode, void *stream) {
  if (!dst || bytes < 16 || grid < 1 || mode < 0 || mode > 2) return 1;
  const hipStream_t s = (hipStream_t)stream;
  if (mode == 0) k_write<<<grid, kThreads, 0, s>>>((u32x4 *)dst, bytes / 16, seed);
  else if (mode == 1) k_write_chunk<false><<<grid, kThreads, 0, s>>>((u32x4 *)dst, bytes / 16, seed);
  else k_write_chunk<true><<<grid, kThreads, 0, s>>>((u32x4 *)dst, bytes / 16, seed);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

// Bytes a chunked read (per 8 blocks of 4 KiB) or write (4 blocks) covers.
int64_t calib_chunk_bytes(int64_t bytes, int grid, int blocks_per_iter) {
  const int64_t it = (int64_t)blocks_per_iter * kThreads;
  return ((bytes / 16) / grid) / it * it * grid * 16;
}

// Mixed read + write: `iters` iterations per workgroup, each reading 8 KiB
// and writing 8 KiB * wpr (wpr 1 .. 8); src must hold grid * iters * 8 KiB
// and dst grid * iters * 8 KiB * wpr (checked against the sizes given).
int calib_mixed(const void *src, int64_t src_bytes, void *dst, int64_t dst_bytes, uint32_t *sink, int grid,
                int64_t iters, int wpr, void *stream) {
  if (!src || !dst || !sink || grid < 1 || iters < 1 || wpr < 1 || wpr > 8) return 1;
  if ((int64_t)grid * iters * 8192 > src_bytes || (int64_t)grid * iters * 8192 * wpr > dst_bytes) return 1;
  const hipStream_t s = (hipStream_t)stream;
  const u32x4 *r = (const u32x4 *)src;
  u32x4 *w = (u32x4 *)dst;
  switch (wpr) {
    case 1: k_mixed<1><<<grid, kThreads, 0, s>>>(r, w, iters, sink); break;
    case 2: k_mixed<2><<<grid, kThreads, 0, s>>>(r, w, iters, sink); break;
    case 3: k_mixed<3><<<grid, kThreads, 0, s>>>(r, w, iters, sink); break;
    case 4: k_mixed<4><<<grid, kThreads, 0, s>>>(r, w, iters, sink); break;
    case 5: k_mixed<5><<<grid, kThreads, 0, s>>>(r, w, iters, sink); break;
    case 6: k_mixed<6><<<grid, kThreads, 0, s>>>(r, w, iters, sink); break;
    case 7: k_mixed<7><<<grid, kThreads, 0, s>>>(r, w, iters, sink); break;
    default: k_mixed<8><<<grid, kThreads, 0, s>>>(r, w, iters, sink); break;
  }
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

// units_per_iter: 1, 2, 4 or 8 units in flight per workgroup.
int calib_gather(const void *pool, int64_t pool_bytes, const int32_t *units, int64_t n_units,
                 uint32_t *sink, int grid, int units_per_iter, void *stream) {
  if (!pool || !units || !sink || grid < 1 || n_units < 1 || pool_bytes < 16) return 1;
  const hipStream_t s = (hipStream_t)stream;
  const int64_t p16 = pool_bytes / 16;
  switch (units_per_iter) {
    case 1: k_gather<1><<<grid, kThreads, 0, s>>>((const u32x4 *)pool, p16, units, n_units, sink); break;
    case 2: k_gather<2><<<grid, kThreads, 0, s>>>((const u32x4 *)pool, p16, units, n_units, sink); break;
    case 4: k_gather<4><<<grid, kThreads, 0, s>>>((const u32x4 *)pool, p16, units, n_units, sink); break;
    case 8: k_gather<8><<<grid, kThreads, 0, s>>>((const u32x4 *)pool, p16, units, n_units, sink); break;
    default: return 1;
  }
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

}  // extern "C"
