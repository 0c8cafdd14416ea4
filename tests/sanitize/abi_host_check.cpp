// Host-only check of the C ABI (exact_io_aware_22_amd/csrc/api.cpp) and of the host side
// of the kernel launchers, built under AddressSanitizer and UndefinedBehaviorSanitizer.
//
// Two builds of this file:
//   - default: the kernel launchers are replaced by stubs that touch no memory. Each stub
//     checks the preconditions the launcher relies on (positive sizes, D in {64, 128},
//     aligned non-NULL pointers, finite positive scale, element counts that fit int64
//     byte offsets) and records the call.
//   - FA_WITH_LAUNCHERS: the real launchers (the .hip sources compiled for the host only)
//     run against stubs of the few HIP runtime calls they make. The launch stub checks
//     every launch configuration (1 <= grid <= 2^31 - 1 workgroups, one-dimensional,
//     whole wavefronts of at most 1024 threads, dynamic LDS within 160 KiB) and records
//     it; the fat binary registration is a no-op, so no device code is needed.
// Either way the program then
//   1. makes calls with known answers: the documented error codes, and what a valid
//      call reaches;
//   2. sweeps every entry point over extreme integer and float arguments (INT_MIN,
//      INT_MAX, powers of two, NaN, infinities, odd addresses), requiring a documented
//      return code, and the checks above whenever a launcher or a launch is reached.
// Any sanitizer report (signed overflow, bad shift, out-of-bounds access, leak) or
// failed check ends the program with a nonzero status.
#include "fa.h"

#include <cfloat>
#include <cinttypes>
#include <climits>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <limits>
#include <string>
#include <vector>

#include "launch.h"

namespace {

int g_failures = 0;
std::string g_last;              // name of the launcher the last call reached, or ""
hipError_t g_status = hipSuccess;  // what the stubs return

#define CHECK(cond)                                                              \
  do {                                                                           \
    if (!(cond)) {                                                               \
      std::fprintf(stderr, "%s:%d: check failed: %s\n", __FILE__, __LINE__, #cond); \
      ++g_failures;                                                              \
    }                                                                            \
  } while (0)

bool al(const void* p, uintptr_t a) { return p && reinterpret_cast<uintptr_t>(p) % a == 0; }

// Exact product of non-negative sizes, in long double (64-bit mantissa on x86).
long double prod(std::initializer_list<long double> xs) {
  long double r = 1;
  for (long double x : xs) r *= x;
  return r;
}

const long double kLimit = std::ldexp(1.0L, 60);  // elements; byte offsets stay in int64

void check_scale(float s) { CHECK(std::isfinite(s) && s > 0.0f); }

[[maybe_unused]] void record(const char* name) {
  CHECK(g_last.empty());  // one launcher per call
  g_last = name;
}

}  // namespace

#ifndef FA_WITH_LAUNCHERS

#define REACHED(r, name) ((r) == (name))

namespace fa {

// Floats of static scratch: m and d padded to 64 floats each, then o_part (the rule the
// header states for fa_decode_noalloc).
int64_t decode_noalloc_floats(int64_t units, int D) {
  return 2 * ((units + 63) / 64 * 64) + units * D;
}

// The chained scans' rule as the header states it: 8 bytes per 2048-element block when a
// row of more than 32 KB has 2 to 64 whole blocks.
int scan_chain_blocks(int n, bool bf16) {
  if (n <= 0 || n % 2048 != 0 || int64_t(n) * (bf16 ? 2 : 4) <= 32768) return 0;
  return n / 2048 >= 2 && n / 2048 <= 64 ? n / 2048 : 0;
}
int64_t scan_workspace_bytes(int64_t rows, int n, bool bf16) {
  return rows * scan_chain_blocks(n, bf16) * 8;
}

static void check_fwd(const FwdArgs& a) {
  CHECK(a.B > 0 && a.H > 0 && a.N > 0 && (a.D == 64 || a.D == 128));
  CHECK(al(a.q, 16) && al(a.k, 16) && al(a.v, 16) && al(a.o, 16) && al(a.lse, 4));
  CHECK(prod({a.cu_seqlens ? 1.0L : a.B, (long double)a.H, (long double)a.N,
              (long double)a.D}) < kLimit);
  check_scale(a.scale);
  CHECK(a.window_left >= -1 && a.window_right >= -1);
  if (a.cu_seqlens) CHECK(al(a.cu_seqlens, 4) && a.max_seqlen > 0);
}
hipError_t launch_fwd_bf16(const FwdArgs& a, hipStream_t) {
  record("fwd_bf16");
  check_fwd(a);
  return g_status;
}
hipError_t launch_fwd_f32(const FwdArgs& a, hipStream_t) {
  record("fwd_f32");
  check_fwd(a);
  CHECK(a.cu_seqlens == nullptr && a.window_left == -1 && a.window_right == -1);
  return g_status;
}

static void check_decode(const DecodeArgs& a, bool scratch_from_library) {
  CHECK(a.B > 0 && a.H > 0 && a.L >= 0 && a.splits >= 1 && (a.D == 64 || a.D == 128));
  CHECK(al(a.q, 16));
  if (a.L > 0) CHECK(al(a.k, 16) && al(a.v, 16));
  if (!scratch_from_library) CHECK(al(a.m, 4) && al(a.d, 4) && al(a.o_part, 16));
  CHECK(prod({(long double)a.B, (long double)a.H, (long double)a.L, (long double)a.D}) < kLimit);
  CHECK(prod({(long double)a.B, (long double)a.H, (long double)a.splits,
              (long double)a.D + 2}) < kLimit);
  check_scale(a.scale);
}
hipError_t launch_decode_partials_bf16(const DecodeArgs& a, hipStream_t) {
  record("decode_bf16");
  check_decode(a, false);
  return g_status;
}
hipError_t launch_decode_partials_f32(const DecodeArgs& a, hipStream_t) {
  record("decode_f32");
  check_decode(a, false);
  return g_status;
}
hipError_t launch_decode_noalloc(const DecodeArgs& a, bool, float* o, float* lse, hipStream_t) {
  record("decode_noalloc");
  check_decode(a, true);
  CHECK(al(o, 16) && al(lse, 4));
  CHECK(decode_noalloc_floats(int64_t(a.B) * a.H * a.splits, a.D) <= kDecodeScratchFloats);
  return g_status;
}

hipError_t launch_combine_partials(const CombineArgs& a, hipStream_t) {
  record("combine");
  CHECK(a.rows > 0 && a.splits >= 1 && (a.D == 64 || a.D == 128));
  CHECK(al(a.m, 4) && al(a.d, 4) && al(a.o_part, 16) && al(a.o, 16) && al(a.lse, 4));
  CHECK(prod({(long double)a.rows, (long double)a.splits, (long double)a.D}) < kLimit);
  return g_status;
}

static void check_bwd(const BwdArgs& a) {
  CHECK(a.B > 0 && a.H > 0 && a.N > 0 && (a.D == 64 || a.D == 128));
  CHECK(al(a.q, 16) && al(a.k, 16) && al(a.v, 16) && al(a.o, 16) && al(a.dout, 16) &&
        al(a.dq, 16) && al(a.dk, 16) && al(a.dv, 16) && al(a.lse, 4) && al(a.delta, 4));
  CHECK(prod({(long double)a.B, (long double)a.H, (long double)a.N, (long double)a.D}) < kLimit);
  check_scale(a.scale);
}
hipError_t launch_bwd_bf16(const BwdArgs& a, hipStream_t) {
  record("bwd_bf16");
  check_bwd(a);
  return g_status;
}
hipError_t launch_bwd_f32(const BwdArgs& a, hipStream_t) {
  record("bwd_f32");
  check_bwd(a);
  return g_status;
}

static void check_rows(const RowReduceArgs& a, bool scan) {
  CHECK(a.rows > 0 && a.n >= 0);
  if (scan) CHECK(a.n > 0 && prod({(long double)a.rows, (long double)a.n, 2.0L}) < kLimit);
  if (a.n > 0) CHECK(al(a.x, a.bf16 ? 2 : 4));
  CHECK(al(a.out0, 4) && al(a.out1, 4));
  // a workspace is passed exactly when the chained path applies by size, aligned
  CHECK(a.max_polls >= 0);
  if (a.slots) CHECK(scan && scan_chain_blocks(a.n, a.bf16) > 0 && al(a.slots, 8));
}
hipError_t launch_softmax_stats(const RowReduceArgs& a, hipStream_t) {
  record("softmax_stats");
  check_rows(a, false);
  return g_status;
}
hipError_t launch_moments(const RowReduceArgs& a, hipStream_t) {
  record("moments");
  check_rows(a, false);
  return g_status;
}
hipError_t launch_softmax_scan(const RowReduceArgs& a, hipStream_t) {
  record("softmax_scan");
  check_rows(a, true);
  return g_status;
}
hipError_t launch_moments_scan(const RowReduceArgs& a, hipStream_t) {
  record("moments_scan");
  check_rows(a, true);
  return g_status;
}

hipError_t launch_calibrate_mfma(float* out, int blocks, int iters, uint32_t, hipStream_t) {
  record("cal_mfma");
  CHECK(al(out, 4) && blocks >= 1 && blocks <= (1 << 20) && iters >= 0);
  return g_status;
}
hipError_t launch_calibrate_overlap(float* out, int blocks, int iters, int mode, hipStream_t) {
  record("cal_overlap");
  CHECK(al(out, 4) && blocks >= 1 && blocks <= (1 << 20) && iters >= 0);
  CHECK(mode >= 0 && mode <= 13 && mode != 7);
  return g_status;
}
hipError_t launch_calibrate_read(const void* x, int64_t nbytes, uint32_t* out, int blocks,
                                 hipStream_t) {
  record("cal_read");
  CHECK(al(out, 4) && blocks >= 1 && blocks <= (1 << 22) && nbytes >= 0 && nbytes % 16 == 0);
  if (nbytes > 0) CHECK(al(x, 16));
  return g_status;
}
hipError_t launch_calibrate_write(void* y, int64_t nbytes, uint32_t, int blocks, hipStream_t) {
  record("cal_write");
  CHECK(al(y, 16) && blocks >= 1 && blocks <= (1 << 22) && nbytes > 0 && nbytes % 16 == 0);
  return g_status;
}
hipError_t launch_calibrate_mix(const void* x, int64_t nbytes, void* y, int ratio, int blocks,
                                hipStream_t) {
  record("cal_mix");
  CHECK(al(x, 16) && al(y, 16) && blocks >= 1 && blocks <= (1 << 22));
  CHECK(nbytes > 0 && nbytes % 4096 == 0 && (ratio == 1 || ratio == 2 || ratio == 4));
  return g_status;
}

}  // namespace fa

#else  // FA_WITH_LAUNCHERS: stubs of the HIP runtime calls the launchers make

#define REACHED(r, name) (!(r).empty())

namespace {
struct LaunchConfig {
  dim3 grid, block;
  size_t shmem = 0;
  hipStream_t stream = nullptr;
};
LaunchConfig g_pushed;
int g_fatbin_handle;
}  // namespace

extern "C" {

void** __hipRegisterFatBinary(const void*) { return reinterpret_cast<void**>(&g_fatbin_handle); }
void __hipUnregisterFatBinary(void**) {}
void __hipRegisterFunction(void**, const void*, char*, const char*, unsigned int, uint3*, uint3*,
                           dim3*, dim3*, int*) {}
void __hipRegisterVar(void**, void*, char*, char*, int, size_t, int, int) {}

hipError_t __hipPushCallConfiguration(dim3 grid, dim3 block, size_t shmem, hipStream_t stream) {
  g_pushed = LaunchConfig{grid, block, shmem, stream};
  return hipSuccess;
}

hipError_t __hipPopCallConfiguration(dim3* grid, dim3* block, size_t* shmem,
                                     hipStream_t* stream) {
  *grid = g_pushed.grid;
  *block = g_pushed.block;
  *shmem = g_pushed.shmem;
  *stream = g_pushed.stream;
  return hipSuccess;
}

hipError_t hipLaunchKernel(const void* fn, dim3 grid, dim3 block, void** args, size_t shmem,
                           hipStream_t) {
  g_last = "launch";  // a call may launch more than one kernel
  CHECK(fn != nullptr && args != nullptr);
  CHECK(grid.x >= 1 && grid.x <= 0x7fffffffu && grid.y == 1 && grid.z == 1);
  CHECK(block.x >= 64 && block.x <= 1024 && block.x % 64 == 0 && block.y == 1 && block.z == 1);
  CHECK(shmem <= 160 * 1024);
  return g_status;
}

hipError_t hipGetLastError(void) { return g_status; }

hipError_t hipGetDevice(int* dev) {
  *dev = 0;
  return hipSuccess;
}

// The static scratch's device address: a fake, 256-byte-aligned, never dereferenced one.
hipError_t hipGetSymbolAddress(void** p, const void*) {
  *p = reinterpret_cast<void*>(uintptr_t(1) << 32);
  return hipSuccess;
}

}  // extern "C"

#endif  // FA_WITH_LAUNCHERS

namespace {

// Fake device addresses: never dereferenced (the stubs touch no memory).
void* const P = reinterpret_cast<void*>(uintptr_t(1) << 20);
float* const F = static_cast<float*>(P);
void* at(uintptr_t off) { return reinterpret_cast<void*>((uintptr_t(1) << 20) + off); }
float* fat(uintptr_t off) { return static_cast<float*>(at(off)); }

// Runs one call and returns its code; `reached` receives the launcher it reached.
template <class Fn>
int run(Fn fn, std::string* reached = nullptr) {
  g_last.clear();
  const int rc = fn();
  if (reached) *reached = g_last;
  CHECK(rc == FA_OK || rc == FA_ERR_NULL || rc == FA_ERR_SHAPE || rc == FA_ERR_DTYPE ||
        rc == FA_ERR_ALIGN || rc == FA_ERR_HIP || rc == FA_ERR_ARG || rc == FA_ERR_SCRATCH);
  // A launcher is reached only by a call that validated; its status maps to OK / HIP.
  if (!g_last.empty()) CHECK(rc == (g_status == hipSuccess ? FA_OK : FA_ERR_HIP));
  if (rc != FA_OK && rc != FA_ERR_HIP) CHECK(g_last.empty());
  return rc;
}

// Sweep calls per entry point that reached a launcher (or, with the real launchers, a
// launch), so the sweep is known to get past validation for every entry point.
std::vector<std::pair<const char*, int>> g_reached;

template <class Fn>
void sweep_call(size_t slot, const char* name, Fn fn) {
  if (g_reached.size() <= slot) g_reached.resize(slot + 1, {name, 0});
  run(fn);
  if (!g_last.empty()) ++g_reached[slot].second;
}

void known_answers() {
  std::string r;
  // forward: codes in the documented order, and what reaches the launcher
  CHECK(run([] { return fa_forward(P, P, P, F, F, 1, 1, 8, 64, 0.125f, 0, FA_BF16, nullptr); },
            &r) == FA_OK && REACHED(r, "fwd_bf16"));
  CHECK(run([] { return fa_forward(P, P, P, F, F, 2, 3, 5, 128, 0.5f, 1, FA_F32, nullptr); },
            &r) == FA_OK && REACHED(r, "fwd_f32"));
  CHECK(run([] { return fa_forward(nullptr, P, P, F, F, 1, 1, 8, 64, 0.1f, 0, 1, nullptr); }) ==
        FA_ERR_NULL);
  CHECK(run([] { return fa_forward(P, P, P, F, F, 1, 1, 8, 96, 0.1f, 0, 1, nullptr); }) ==
        FA_ERR_SHAPE);
  CHECK(run([] { return fa_forward(P, P, P, F, F, 1, 1, 8, 64, 0.1f, 0, 9, nullptr); }) ==
        FA_ERR_DTYPE);
  CHECK(run([] { return fa_forward(at(8), P, P, F, F, 1, 1, 8, 64, 0.1f, 0, 1, nullptr); }) ==
        FA_ERR_ALIGN);
  CHECK(run([] { return fa_forward(P, P, P, F, F, 1, 1, 8, 64, NAN, 0, 1, nullptr); }) ==
        FA_ERR_ARG);
  CHECK(run([] { return fa_forward(P, P, P, F, F, 1, 1, 8, 64, 0.1f, 2, 1, nullptr); }) ==
        FA_ERR_ARG);
  CHECK(run([] {
          return fa_forward(nullptr, nullptr, nullptr, nullptr, nullptr, 0, 1, 8, 64, 0.1f, 0, 1,
                            nullptr);
        }) == FA_OK);
  CHECK(run([] {
          return fa_forward(P, P, P, F, F, 1 << 30, 1 << 30, 1 << 30, 64, 0.1f, 0, 1, nullptr);
        }) == FA_ERR_SHAPE);
  // forward_ext: windows and packed sequences need bf16; the packed size check is H x N x D
  CHECK(run([] {
          return fa_forward_ext(P, P, P, F, F, 1, 1, 8, 64, 0.1f, 0, 3, -1, nullptr, 0, FA_F32,
                                nullptr);
        }) == FA_ERR_DTYPE);
  CHECK(run([] {
          return fa_forward_ext(P, P, P, F, F, 1 << 30, 4, 1024, 64, 0.1f, 0, -1, -1,
                                static_cast<const int*>(P), 0, 1, nullptr);
        }) == FA_OK);
  CHECK(run([] {
          return fa_forward_ext(P, P, P, F, F, 1, 1, 8, 64, 0.1f, 0, -2, -1, nullptr, 0, 1,
                                nullptr);
        }) == FA_ERR_ARG);
  CHECK(run([] {
          return fa_forward_ext(P, P, P, F, F, 3, 2, 100, 64, 0.1f, 1, 7, 0,
                                static_cast<const int*>(at(4)), 40, 1, nullptr);
        },
            &r) == FA_OK && REACHED(r, "fwd_bf16"));
  // decode, combine, noalloc
  CHECK(run([] { return fa_decode_partials(P, P, P, F, F, F, 1, 1, 64, 128, 0.1f, 4, 1, nullptr); },
            &r) == FA_OK && REACHED(r, "decode_bf16"));
  CHECK(run([] {
          return fa_decode_partials(P, nullptr, nullptr, F, F, F, 1, 1, 0, 64, 0.1f, 4, 0, nullptr);
        },
            &r) == FA_OK && REACHED(r, "decode_f32"));
  CHECK(run([] {
          return fa_decode_partials(nullptr, P, P, F, F, F, 1, 1, 0, 64, 0.1f, 4, 0, nullptr);
        }) == FA_ERR_NULL);
  CHECK(run([] { return fa_combine_partials(F, F, F, 4, 3, 64, F, F, nullptr); }, &r) == FA_OK &&
        REACHED(r, "combine"));
  CHECK(run([] { return fa_combine_partials(F, F, fat(4), 4, 3, 64, F, F, nullptr); }) ==
        FA_ERR_ALIGN);
  CHECK(run([] { return fa_decode_noalloc(P, P, P, F, F, 16, 32, 32768, 128, 0.1f, 64, 1, nullptr); },
            &r) == FA_OK && REACHED(r, "decode_noalloc"));
  CHECK(run([] { return fa_decode_noalloc(P, P, P, F, F, 16, 32, 1, 128, 0.1f, 1024, 1, nullptr); }) ==
        FA_ERR_SCRATCH);
  CHECK(run([] {
          return fa_decode_noalloc(P, P, P, F, F, INT_MAX, INT_MAX, 1, 64, 0.1f, INT_MAX, 1,
                                   nullptr);
        }) == FA_ERR_SHAPE);
  // backward and the row kernels
  CHECK(run([] {
          return fa_backward(P, P, P, F, F, P, F, F, F, F, 1, 2, 8, 128, 0.1f, 1, 1, nullptr);
        },
            &r) == FA_OK && REACHED(r, "bwd_bf16"));
  CHECK(run([] {
          return fa_backward(P, P, P, F, F, P, fat(2), F, F, F, 1, 2, 8, 128, 0.1f, 1, 1, nullptr);
        }) == FA_ERR_ALIGN);
  CHECK(run([] { return fa_softmax_stats(at(2), F, F, 4, 100, FA_BF16, nullptr); }, &r) == FA_OK &&
        REACHED(r, "softmax_stats"));
  CHECK(run([] { return fa_moments(at(2), F, F, 4, 100, FA_F32, nullptr); }) == FA_ERR_ALIGN);
  CHECK(run([] { return fa_moments(nullptr, F, F, 4, 0, FA_F32, nullptr); }, &r) == FA_OK &&
        REACHED(r, "moments"));  // n = 0: x is never read
  CHECK(run([] { return fa_softmax_scan(P, F, F, 1 << 30, 1 << 30, 0, nullptr); }) ==
        FA_ERR_SHAPE);
  CHECK(run([] { return fa_moments_scan(P, F, F, 3, 5000, 1, nullptr); }, &r) == FA_OK &&
        REACHED(r, "moments_scan"));
  // calibration kernels
  CHECK(run([] { return fa_calibrate_mix(P, 4096, P, 2, 8, nullptr); }, &r) == FA_OK &&
        REACHED(r, "cal_mix"));
  CHECK(run([] { return fa_calibrate_write(nullptr, 0, 1, 4, nullptr); }, &r) == FA_OK &&
        r.empty());
  CHECK(run([] { return fa_calibrate_read(nullptr, 0, static_cast<unsigned*>(P), 4, nullptr); },
            &r) == FA_OK && REACHED(r, "cal_read"));
  CHECK(run([] { return fa_calibrate_overlap(F, 4, 1, 7, nullptr); }) == FA_ERR_ARG);
  // a launcher's failure becomes FA_ERR_HIP
  g_status = hipErrorInvalidValue;
  CHECK(run([] { return fa_forward(P, P, P, F, F, 1, 1, 8, 64, 0.1f, 0, 1, nullptr); }) ==
        FA_ERR_HIP);
  g_status = hipSuccess;
  // strerror covers every code and unknown ones
  for (int c : {0, -1, -2, -3, -4, -5, -6, -7, -8, 1, INT_MIN, INT_MAX})
    CHECK(fa_strerror(c) != nullptr && std::strlen(fa_strerror(c)) > 0);
  CHECK(fa_abi_version() == 2);
}

// Extreme values for the sweep.
const std::vector<int> kInts = {INT_MIN, -2, -1, 0, 1, 2, 3, 63, 64, 65, 127, 128, 4096,
                                1 << 20, (1 << 22) + 1, 1 << 30, INT_MAX};
const std::vector<int> kDims = {INT_MIN, -1, 0, 32, 64, 96, 128, 256, INT_MAX};
const std::vector<float> kScales = {0.125f, 0.0f, -1.0f, NAN, INFINITY, -INFINITY,
                                    std::numeric_limits<float>::denorm_min(), FLT_MAX};
const std::vector<long long> kBytes = {LLONG_MIN, -4096, -16, 0, 16, 1000, 4096, 8192,
                                       int64_t(1) << 40, LLONG_MAX};
const std::vector<uintptr_t> kOffsets = {0, 1, 2, 4, 8};

void* ptr(int i) { return i < 0 ? nullptr : at(kOffsets[i % kOffsets.size()]); }

uint64_t g_rng = 0x9e3779b97f4a7c15ull;
uint64_t next() {  // splitmix64
  uint64_t z = (g_rng += 0x9e3779b97f4a7c15ull);
  z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
  z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
  return z ^ (z >> 31);
}
int pick_int() { return kInts[next() % kInts.size()]; }
int pick_dim() { return kDims[next() % kDims.size()]; }
float pick_scale() { return kScales[next() % kScales.size()]; }
// Mostly aligned addresses, sometimes NULL or misaligned.
void* pick_ptr() {
  const uint64_t r = next() % 16;
  if (r == 0) return nullptr;
  if (r == 1) return ptr(1 + int(next() % 4));
  return P;
}
float* pick_fptr() { return static_cast<float*>(pick_ptr()); }

void sweep(int iterations) {
  for (int it = 0; it < iterations; ++it) {
    const int B = pick_int(), H = pick_int(), N = pick_int(), D = pick_dim(), dt = pick_int() % 3;
    const int c = int(next() % 4) - 1, wl = pick_int(), wr = pick_int(), ms = pick_int();
    const int splits = pick_int(), rows = pick_int(), n = pick_int();
    const float sc = pick_scale();
    const long long nb = kBytes[next() % kBytes.size()];
    const int blocks = pick_int(), iters = pick_int(), mode = pick_int(), ratio = pick_int();
    const int* cu = (next() % 2) ? static_cast<const int*>(pick_ptr()) : nullptr;
    sweep_call(0, "fa_forward", [&] { return fa_forward(pick_ptr(), pick_ptr(), pick_ptr(), pick_fptr(), pick_fptr(), B, H,
                                N, D, sc, c, dt, nullptr); });
    sweep_call(1, "fa_forward_ext", [&] { return fa_forward_ext(pick_ptr(), pick_ptr(), pick_ptr(), pick_fptr(), pick_fptr(),
                                    B, H, N, D, sc, c, wl, wr, cu, ms, dt, nullptr); });
    sweep_call(2, "fa_decode_partials", [&] { return fa_decode_partials(pick_ptr(), pick_ptr(), pick_ptr(), pick_fptr(),
                                        pick_fptr(), pick_fptr(), B, H, N, D, sc, splits, dt,
                                        nullptr); });
    sweep_call(3, "fa_decode_noalloc", [&] { return fa_decode_noalloc(pick_ptr(), pick_ptr(), pick_ptr(), pick_fptr(),
                                       pick_fptr(), B, H, N, D, sc, splits, dt, nullptr); });
    sweep_call(4, "fa_combine_partials", [&] { return fa_combine_partials(pick_fptr(), pick_fptr(), pick_fptr(), splits, rows, D,
                                         pick_fptr(), pick_fptr(), nullptr); });
    sweep_call(5, "fa_backward", [&] { return fa_backward(pick_ptr(), pick_ptr(), pick_ptr(), pick_fptr(), pick_fptr(),
                                 pick_ptr(), pick_fptr(), pick_fptr(), pick_fptr(), pick_fptr(), B,
                                 H, N, D, sc, c, dt, nullptr); });
    sweep_call(6, "fa_softmax_stats", [&] { return fa_softmax_stats(pick_ptr(), pick_fptr(), pick_fptr(), rows, n, dt, nullptr); });
    sweep_call(7, "fa_moments", [&] { return fa_moments(pick_ptr(), pick_fptr(), pick_fptr(), rows, n, dt, nullptr); });
    sweep_call(8, "fa_softmax_scan", [&] { return fa_softmax_scan(pick_ptr(), pick_fptr(), pick_fptr(), rows, n, dt, nullptr); });
    sweep_call(9, "fa_moments_scan", [&] { return fa_moments_scan(pick_ptr(), pick_fptr(), pick_fptr(), rows, n, dt, nullptr); });
    const int polls = pick_int();
    sweep_call(15, "fa_softmax_scan_ws", [&] { return fa_softmax_scan_ws(pick_ptr(), pick_fptr(), pick_fptr(), rows, n, dt,
                                        pick_ptr(), nb, polls, nullptr); });
    sweep_call(16, "fa_moments_scan_ws", [&] { return fa_moments_scan_ws(pick_ptr(), pick_fptr(), pick_fptr(), rows, n, dt,
                                        pick_ptr(), nb, polls, nullptr); });
    {
      const long long w = fa_scan_workspace_bytes(rows, n, dt);
      CHECK(w == -1 || w == int64_t(rows) * fa::scan_chain_blocks(n, dt == 1) * 8);
    }
    sweep_call(10, "fa_calibrate_mfma", [&] { return fa_calibrate_mfma(pick_fptr(), blocks, iters, unsigned(it), nullptr); });
    sweep_call(11, "fa_calibrate_overlap", [&] { return fa_calibrate_overlap(pick_fptr(), blocks, iters, mode, nullptr); });
    sweep_call(12, "fa_calibrate_read", [&] { return fa_calibrate_read(pick_ptr(), nb, static_cast<unsigned*>(pick_ptr()), blocks,
                                       nullptr); });
    sweep_call(13, "fa_calibrate_write", [&] { return fa_calibrate_write(pick_ptr(), nb, 7u, blocks, nullptr); });
    sweep_call(14, "fa_calibrate_mix", [&] { return fa_calibrate_mix(pick_ptr(), nb, pick_ptr(), ratio, blocks, nullptr); });
  }
}

}  // namespace

int main(int argc, char** argv) {
  const int iterations = argc > 1 ? std::atoi(argv[1]) : 200000;
  known_answers();
  sweep(iterations);
  for (const auto& [name, count] : g_reached) {
    std::printf("%-22s reached a launch in %d sweep calls\n", name, count);
    if (iterations >= 100000) CHECK(count >= 100);
  }
  if (g_failures) {
    std::fprintf(stderr, "%d check(s) failed\n", g_failures);
    return 1;
  }
  std::printf("abi host check: %d sweep iterations, all checks passed\n", iterations);
  return 0;
}
