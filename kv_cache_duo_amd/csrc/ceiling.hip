// Measured hardware ceilings used as a second reference next to the vendor
// peaks when the kernels' roofline fractions are reported:
//   ceiling stream_read <MiB>  -- 16-byte streaming reads of a buffer (HBM)
//   ceiling stream_read_rotating <MiB> <n> -- the same over n buffers in turn
//   ceiling copy <MiB>         -- a plain device copy of <MiB> (reads and writes
//                                 <MiB> each, 16 bytes per lane): the known
//                                 traffic that calibrates FETCH_SIZE / WRITE_SIZE
//   ceiling mfma               -- back-to-back v_mfma_f32_32x32x16_bf16
//   ceiling mfma_random        -- the same with changing pseudo-random operands
//   ceiling mfma_fp8_random    -- v_mfma_scale_f32_32x32x64_f8f6f4 (e4m3, unit
//                                 scales) with changing pseudo-random operands
//   ceiling lds_read           -- conflict-free 16-byte LDS reads (ds_read_b128),
//                                 8 in flight per wave, 8 work-groups per CU;
//                                 bytes per CU per shader clock
// Standalone executable (not part of the C ABI); prints one JSON line.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>
#include <cstring>

namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;

constexpr size_t kSlab = 4096;  // 16-byte elements per block (64 KB)

// Each block reads one contiguous 64 KB slab, 4 loads in flight per thread.
template <bool NT>
__global__ __launch_bounds__(256) void stream_read(const u32x4* __restrict__ p, unsigned* out) {
  const size_t base = (size_t)blockIdx.x * kSlab;
  unsigned acc = 0;
  for (size_t i = threadIdx.x; i < kSlab; i += 256 * 4) {
    u32x4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const size_t idx = base + i + (size_t)u * 256;
      v[u] = NT ? __builtin_nontemporal_load(p + idx) : p[idx];
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  if (acc == 0x9e3779b9u) out[blockIdx.x] = acc;  // keeps the loads; practically never true
}

// Each block copies one contiguous 64 KB slab, 4 loads in flight per thread.
__global__ __launch_bounds__(256) void copy_slabs(const u32x4* __restrict__ src, u32x4* __restrict__ dst) {
  const size_t base = (size_t)blockIdx.x * kSlab;
  for (size_t i = threadIdx.x; i < kSlab; i += 256 * 4) {
    u32x4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = src[base + i + (size_t)u * 256];
#pragma unroll
    for (int u = 0; u < 4; ++u) dst[base + i + (size_t)u * 256] = v[u];
  }
}

// 4 independent accumulators per wave, `iters` rounds of 4 MFMAs each.
__global__ __launch_bounds__(256) void mfma_loop(float* out, int iters) {
  bf16x8 a, b;
  for (int j = 0; j < 8; ++j) {
    a[j] = (__bf16)(0.001f * (threadIdx.x + j));
    b[j] = (__bf16)(0.002f * (threadIdx.x - j));
  }
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int i = 0; i < iters; ++i) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
  }
  float s = 0.f;
  for (int r = 0; r < 16; ++r) s += c0[r] + c1[r] + c2[r] + c3[r];
  if (s == 1234.5f) out[blockIdx.x] = s;
}

// The same with operands that change from one MFMA to the next: 4 A and 4 B
// fragments of pseudo-random bf16 values (uniform in [-2, 2), as attention
// inputs of unit variance), paired differently by every MFMA of a round.
// The MFMA rate under sustained load is power-limited, and constant operands
// switch far fewer bits than real data.
__device__ __forceinline__ float hash_unit(unsigned x) {
  x ^= x >> 16; x *= 0x7feb352du; x ^= x >> 15; x *= 0x846ca68bu; x ^= x >> 16;
  return (float)(x >> 8) * (4.0f / 16777216.0f) - 2.0f;
}
__global__ __launch_bounds__(256) void mfma_loop_random(float* out, int iters) {
  bf16x8 a[4], b[4];
  const unsigned seed = (blockIdx.x * 256u + threadIdx.x) * 64u;
#pragma unroll
  for (int f = 0; f < 4; ++f)
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      a[f][j] = (__bf16)hash_unit(seed + f * 8 + j);
      b[f][j] = (__bf16)hash_unit(seed + 32 + f * 8 + j);
    }
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int i = 0; i < iters; i += 4) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[0], b[0], c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[1], b[1], c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[2], b[2], c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[3], b[3], c3, 0, 0, 0);
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[1], b[2], c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[2], b[3], c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[3], b[0], c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[0], b[1], c3, 0, 0, 0);
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[2], b[0], c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[3], b[1], c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[0], b[2], c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[1], b[3], c3, 0, 0, 0);
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[3], b[3], c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[0], b[0], c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[1], b[1], c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[2], b[2], c3, 0, 0, 0);
  }
  float s = 0.f;
  for (int r = 0; r < 16; ++r) s += c0[r] + c1[r] + c2[r] + c3[r];
  if (s == 1234.5f) out[blockIdx.x] = s;
}

typedef int i32x8 __attribute__((ext_vector_type(8)));
// The same rounds on e4m3 operands (pseudo-random values in [-2, 2) as
// codes), through the scaled fp8 instruction with unit scales (E8M0 127).
__device__ __forceinline__ int fp8_word(unsigned seed) {
  const unsigned w = __builtin_amdgcn_cvt_pk_fp8_f32(hash_unit(seed), hash_unit(seed + 1), 0u, false);
  return (int)__builtin_amdgcn_cvt_pk_fp8_f32(hash_unit(seed + 2), hash_unit(seed + 3), w, true);
}
#define FP8_MFMA(A, B, C) __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(A, B, C, 0, 0, 0, 127, 0, 127)
__global__ __launch_bounds__(256) void mfma_loop_fp8_random(float* out, int iters) {
  i32x8 a[4], b[4];
  const unsigned seed = (blockIdx.x * 256u + threadIdx.x) * 512u;
#pragma unroll
  for (int f = 0; f < 4; ++f)
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      a[f][j] = fp8_word(seed + f * 32 + 4 * j);
      b[f][j] = fp8_word(seed + 256 + f * 32 + 4 * j);
    }
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int i = 0; i < iters; i += 4) {
    c0 = FP8_MFMA(a[0], b[0], c0); c1 = FP8_MFMA(a[1], b[1], c1);
    c2 = FP8_MFMA(a[2], b[2], c2); c3 = FP8_MFMA(a[3], b[3], c3);
    c0 = FP8_MFMA(a[1], b[2], c0); c1 = FP8_MFMA(a[2], b[3], c1);
    c2 = FP8_MFMA(a[3], b[0], c2); c3 = FP8_MFMA(a[0], b[1], c3);
    c0 = FP8_MFMA(a[2], b[0], c0); c1 = FP8_MFMA(a[3], b[1], c1);
    c2 = FP8_MFMA(a[0], b[2], c2); c3 = FP8_MFMA(a[1], b[3], c3);
    c0 = FP8_MFMA(a[3], b[3], c0); c1 = FP8_MFMA(a[0], b[0], c1);
    c2 = FP8_MFMA(a[1], b[1], c2); c3 = FP8_MFMA(a[2], b[2], c3);
  }
  float s = 0.f;
  for (int r = 0; r < 16; ++r) s += c0[r] + c1[r] + c2[r] + c3[r];
  if (s == 1234.5f) out[blockIdx.x] = s;
}
#undef FP8_MFMA

bool ok(hipError_t e, const char* what) {
  if (e != hipSuccess) fprintf(stderr, "%s: %s\n", what, hipGetErrorString(e));
  return e == hipSuccess;
}

int run_stream_read(size_t mib) {
  const size_t bytes = mib << 20;
  const unsigned blocks = (unsigned)(bytes / 16 / kSlab);
  if (blocks == 0) return 2;
  u32x4* p = nullptr;
  unsigned* out = nullptr;
  if (!ok(hipMalloc(&p, (size_t)blocks * kSlab * 16), "hipMalloc") || !ok(hipMalloc(&out, blocks * 4), "hipMalloc"))
    return 1;
  if (!ok(hipMemset(p, 1, (size_t)blocks * kSlab * 16), "hipMemset")) return 1;
  hipEvent_t a, b;
  if (!ok(hipEventCreate(&a), "event") || !ok(hipEventCreate(&b), "event")) return 1;
  const int reps = bytes < ((size_t)1 << 30) ? 50 : 5;
  double gbs[2];
  for (int nt = 0; nt < 2; ++nt) {
    auto k = nt ? stream_read<true> : stream_read<false>;
    for (int w = 0; w < 2; ++w) hipLaunchKernelGGL(k, dim3(blocks), dim3(256), 0, 0, p, out);
    (void)hipEventRecord(a, 0);
    for (int r = 0; r < reps; ++r) hipLaunchKernelGGL(k, dim3(blocks), dim3(256), 0, 0, p, out);
    (void)hipEventRecord(b, 0);
    if (!ok(hipEventSynchronize(b), "sync")) return 1;
    float ms = 0.f;
    (void)hipEventElapsedTime(&ms, a, b);
    gbs[nt] = (double)reps * blocks * kSlab * 16 / (ms * 1e-3) / 1e9;
  }
  printf("{\"ceiling\": \"stream_read\", \"mib\": %zu, \"plain_gbs\": %.1f, \"nontemporal_gbs\": %.1f}\n", mib, gbs[0],
         gbs[1]);
  return 0;
}

// A copy of `mib` MiB, launched 3 times (FETCH_SIZE / WRITE_SIZE calibration:
// each launch reads and writes exactly mib MiB).
int run_copy(size_t mib) {
  const size_t bytes = mib << 20;
  const unsigned blocks = (unsigned)(bytes / 16 / kSlab);
  if (blocks == 0 || (size_t)blocks * kSlab * 16 != bytes) return 2;
  u32x4 *src = nullptr, *dst = nullptr;
  if (!ok(hipMalloc(&src, bytes), "hipMalloc") || !ok(hipMalloc(&dst, bytes), "hipMalloc")) return 1;
  if (!ok(hipMemset(src, 1, bytes), "hipMemset")) return 1;
  hipEvent_t a, b;
  if (!ok(hipEventCreate(&a), "event") || !ok(hipEventCreate(&b), "event")) return 1;
  (void)hipEventRecord(a, 0);
  for (int r = 0; r < 3; ++r) hipLaunchKernelGGL(copy_slabs, dim3(blocks), dim3(256), 0, 0, src, dst);
  (void)hipEventRecord(b, 0);
  if (!ok(hipEventSynchronize(b), "sync")) return 1;
  float ms = 0.f;
  (void)hipEventElapsedTime(&ms, a, b);
  printf("{\"ceiling\": \"copy\", \"mib\": %zu, \"launches\": 3, \"read_write_gbs\": %.1f}\n", mib,
         3.0 * 2.0 * bytes / (ms * 1e-3) / 1e9);
  return 0;
}

// One launch per buffer of `nbuf` separate buffers of `mib` MiB each, in
// turn, so no launch finds its data in the 256 MB Infinity Cache: the rate
// one launch of that size gets from HBM, launch ramp and drain included.
int run_stream_read_rotating(size_t mib, int nbuf) {
  const size_t bytes = mib << 20;
  const unsigned blocks = (unsigned)(bytes / 16 / kSlab);
  if (blocks == 0 || nbuf < 1 || nbuf > 64) return 2;
  u32x4* p[64] = {};
  unsigned* out = nullptr;
  for (int i = 0; i < nbuf; ++i) {
    if (!ok(hipMalloc(&p[i], (size_t)blocks * kSlab * 16), "hipMalloc")) return 1;
    if (!ok(hipMemset(p[i], 1, (size_t)blocks * kSlab * 16), "hipMemset")) return 1;
  }
  if (!ok(hipMalloc(&out, blocks * 4), "hipMalloc")) return 1;
  hipEvent_t a, b;
  if (!ok(hipEventCreate(&a), "event") || !ok(hipEventCreate(&b), "event")) return 1;
  const int launches = 16 * nbuf;
  for (int i = 0; i < nbuf; ++i) hipLaunchKernelGGL(stream_read<true>, dim3(blocks), dim3(256), 0, 0, p[i], out);
  (void)hipEventRecord(a, 0);
  for (int r = 0; r < launches; ++r)
    hipLaunchKernelGGL(stream_read<true>, dim3(blocks), dim3(256), 0, 0, p[r % nbuf], out);
  (void)hipEventRecord(b, 0);
  if (!ok(hipEventSynchronize(b), "sync")) return 1;
  float ms = 0.f;
  (void)hipEventElapsedTime(&ms, a, b);
  const double us = ms * 1e3 / launches;
  printf("{\"ceiling\": \"stream_read_rotating\", \"mib\": %zu, \"buffers\": %d, \"us_per_launch\": %.2f, "
         "\"nontemporal_gbs\": %.1f}\n",
         mib, nbuf, us, (double)blocks * kSlab * 16 / us / 1e3);
  for (int i = 0; i < nbuf; ++i) (void)hipFree(p[i]);
  (void)hipFree(out);
  return 0;
}

// Each wave reads 1 KB rows of a 16 KB LDS buffer (64 lanes x 16 contiguous
// bytes: no bank conflicts), 8 reads per round. The row offset passes through
// an empty asm statement every round, so the compiler can neither hoist nor
// merge the reads. Block 0 stamps the shader clock and the 100 MHz real-time
// counter around its loop: their ratio is the clock the reads ran at. (Its
// own loop ends early -- the oldest waves of a CU are served first -- so the
// rate itself comes from the launch's event time.)
__global__ __launch_bounds__(256) void lds_read(unsigned* out, int iters) {
  __shared__ u32x4 buf[1024];
  for (unsigned i = threadIdx.x; i < 1024; i += 256) buf[i] = u32x4{i, 3 * i + 1, 5 * i + 2, 7 * i + 3};
  __syncthreads();
  const unsigned lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  unsigned off = wave * 256 + lane;
  u32x4 acc = {0u, 0u, 0u, 0u};
  const unsigned long long t0 = __builtin_readcyclecounter();
  const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int j = 0; j < 8; ++j) acc ^= buf[(off + 128 * j) & 1023];
    asm volatile("" : "+v"(off));
  }
  const unsigned long long t1 = __builtin_readcyclecounter();
  const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
  if ((acc.x ^ acc.y ^ acc.z ^ acc.w) == 0x9e3779b9u) out[4 + blockIdx.x] = acc.x;
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    out[0] = (unsigned)(t1 - t0);
    out[1] = (unsigned)(r1 - r0);
  }
}

// mode 0: bf16 constant operands, 1: bf16 random operands, 2: fp8 random
int run_mfma(int mode) {
  int dev = 0, cus = 0;
  if (!ok(hipGetDevice(&dev), "device") ||
      !ok(hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev), "attr"))
    return 1;
  const unsigned blocks = (unsigned)cus * 8;  // 8 work-groups of 4 waves per CU
  const int iters = 4096;
  float* out = nullptr;
  if (!ok(hipMalloc(&out, blocks * 4), "hipMalloc")) return 1;
  hipEvent_t a, b;
  if (!ok(hipEventCreate(&a), "event") || !ok(hipEventCreate(&b), "event")) return 1;
  auto kernel = mode == 2 ? mfma_loop_fp8_random : mode == 1 ? mfma_loop_random : mfma_loop;
  hipLaunchKernelGGL(kernel, dim3(blocks), dim3(256), 0, 0, out, iters);
  (void)hipEventRecord(a, 0);
  const int reps = 5;
  for (int r = 0; r < reps; ++r) hipLaunchKernelGGL(kernel, dim3(blocks), dim3(256), 0, 0, out, iters);
  (void)hipEventRecord(b, 0);
  if (!ok(hipEventSynchronize(b), "sync")) return 1;
  float ms = 0.f;
  (void)hipEventElapsedTime(&ms, a, b);
  const double per_mfma = mode == 2 ? 2.0 * 32 * 32 * 64 : 2.0 * 32 * 32 * 16;
  const double flop = (double)reps * blocks * 4 /*waves*/ * iters * 4 /*mfma*/ * per_mfma;
  const char* name = mode == 2 ? "mfma_fp8_32x32x64_random_operands"
                     : mode == 1 ? "mfma_bf16_32x32x16_random_operands" : "mfma_bf16_32x32x16";
  printf("{\"ceiling\": \"%s\", \"cus\": %d, \"tflops\": %.1f}\n", name, cus, flop / (ms * 1e-3) / 1e12);
  return 0;
}

// LDS read rate: bytes per CU per shader clock, and in TB/s over the chip.
int run_lds_read() {
  int dev = 0, cus = 0;
  if (!ok(hipGetDevice(&dev), "device") ||
      !ok(hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev), "attr"))
    return 1;
  const unsigned blocks = (unsigned)cus * 8;  // 8 work-groups of 4 waves per CU, all resident
  const int iters = 1 << 14;
  unsigned* out = nullptr;
  if (!ok(hipMalloc(&out, (4 + blocks) * sizeof(unsigned)), "hipMalloc")) return 1;
  hipEvent_t a, b;
  if (!ok(hipEventCreate(&a), "event") || !ok(hipEventCreate(&b), "event")) return 1;
  hipLaunchKernelGGL(lds_read, dim3(blocks), dim3(256), 0, 0, out, iters);
  (void)hipEventRecord(a, 0);
  hipLaunchKernelGGL(lds_read, dim3(blocks), dim3(256), 0, 0, out, iters);
  (void)hipEventRecord(b, 0);
  if (!ok(hipEventSynchronize(b), "sync")) return 1;
  float ms = 0.f;
  (void)hipEventElapsedTime(&ms, a, b);
  unsigned stamps[2] = {0, 0};
  if (!ok(hipMemcpy(stamps, out, sizeof(stamps), hipMemcpyDeviceToHost), "copy")) return 1;
  const double bytes_per_cu = 8.0 * 256 * iters * 8 * 16;  // per CU: 8 blocks x 256 lanes x reads x 16 B
  const double clock_ghz = stamps[1] ? (double)stamps[0] / stamps[1] * 0.1 : 0.0;  // real-time counter: 100 MHz
  const double seconds = ms * 1e-3;
  printf("{\"ceiling\": \"lds_read_b128\", \"cus\": %d, \"bytes_per_cu_per_clock\": %.1f, \"clock_ghz\": %.3f, "
         "\"tbs\": %.1f}\n", cus, clock_ghz > 0 ? bytes_per_cu / (seconds * clock_ghz * 1e9) : 0.0, clock_ghz,
         bytes_per_cu * cus / seconds / 1e12);
  return 0;
}

}  // namespace

int main(int argc, char** argv) {
  if (argc >= 2 && std::strcmp(argv[1], "stream_read") == 0)
    return run_stream_read(argc >= 3 ? (size_t)std::atoll(argv[2]) : 4096);
  if (argc >= 2 && std::strcmp(argv[1], "stream_read_rotating") == 0)
    return run_stream_read_rotating(argc >= 3 ? (size_t)std::atoll(argv[2]) : 132, argc >= 4 ? std::atoi(argv[3]) : 8);
  if (argc >= 2 && std::strcmp(argv[1], "copy") == 0) return run_copy(argc >= 3 ? (size_t)std::atoll(argv[2]) : 1024);
  if (argc >= 2 && std::strcmp(argv[1], "mfma") == 0) return run_mfma(0);
  if (argc >= 2 && std::strcmp(argv[1], "mfma_random") == 0) return run_mfma(1);
  if (argc >= 2 && std::strcmp(argv[1], "mfma_fp8_random") == 0) return run_mfma(2);
  if (argc >= 2 && std::strcmp(argv[1], "lds_read") == 0) return run_lds_read();
  fprintf(stderr, "usage: ceiling stream_read <MiB> | ceiling stream_read_rotating <MiB> <buffers> | ceiling copy <MiB>"
                  " | ceiling mfma"
                  " | ceiling mfma_random | ceiling mfma_fp8_random | ceiling lds_read\n");
  return 2;
}
