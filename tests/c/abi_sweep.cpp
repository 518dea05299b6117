// Host-side validation sweep of the C ABI: a seeded random mix of calls to
// every entry point with extreme sizes (negative, zero, at and past each
// limit, INT64_MAX), null, misaligned and aligned fake pointers and any
// workspace size, against a library whose host code is built with the
// address and undefined-behaviour sanitizers: validation must never
// overflow, read out of bounds or return a status the ABI does not define.
// Only for a machine without a GPU: the few calls that pass validation
// reach a launch on fake pointers, which the runtime then refuses.
//
//   abi_sweep SEED ITERS
#include <climits>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <random>

#include "epdc.h"

namespace {

std::mt19937_64 rng;

template <typename T, size_t N>
T pick(const T (&v)[N]) {
  return v[rng() % N];
}

const int64_t kI64[] = {-1, 0, 1, 7, 255, 256, 4097, 16384, (1LL << 30) - 1, 1LL << 30,
                        1LL << 31, INT64_MAX, INT64_MIN};
const int kI32[] = {-1, 0, 1, 2, 7, 8, 16, 17, 32, 128, 1024, 1025, 7168, 8192, 65536,
                    INT_MAX, INT_MIN};
const size_t kSizes[] = {0, 1, 255, 256, 4096, size_t(1) << 20, SIZE_MAX};

void* ptr() {
  static void* const p[] = {nullptr, (void*)0x10000, (void*)0x10002, (void*)0x10004,
                            (void*)0x10008, (void*)0x10100};
  return pick(p);
}
template <typename T>
T* p() {
  return static_cast<T*>(ptr());
}

}  // namespace

int main(int argc, char** argv) {
  if (argc != 3) {
    std::fprintf(stderr, "usage: %s SEED ITERS\n", argv[0]);
    return 1;
  }
  // The calls that pass validation launch kernels on fake pointers, which
  // only a machine without a GPU refuses harmlessly: never run with one.
  int devices = 0;
  if (hipGetDeviceCount(&devices) == hipSuccess && devices > 0) {
    std::fprintf(stderr, "abi_sweep: %d GPU(s) visible; this sweep runs only without a GPU\n",
                 devices);
    return 2;
  }
  rng.seed(std::strtoull(argv[1], nullptr, 10));
  const long iters = std::strtol(argv[2], nullptr, 10);
  long rejected = 0, passed = 0;
  for (long it = 0; it < iters; ++it) {
    int st = EP_OK;
    switch (it % 9) {
      case 0:
        st = ep_compute_send_counts(p<const int64_t>(), pick(kI64), pick(kI32), pick(kI32),
                                    pick(kI32), pick(kI32), p<int32_t>(), p<uint8_t>(),
                                    p<int32_t>(), p<int32_t>(), p<int32_t>(), ptr(),
                                    pick(kSizes), nullptr);
        break;
      case 1:
        st = ep_build_send_layout(p<const int64_t>(), p<const float>(), p<const int32_t>(),
                                  p<const int32_t>(), pick(kI64), pick(kI32), pick(kI32),
                                  pick(kI32), pick(kI64), p<int32_t>(), p<int32_t>(),
                                  p<int32_t>(), p<float>(), p<int32_t>(), ptr(), pick(kSizes),
                                  nullptr);
        break;
      case 2:
        st = ep_dispatch_layout(p<const int64_t>(), p<const float>(), pick(kI64), pick(kI32),
                                pick(kI32), pick(kI32), pick(kI64), p<int32_t>(), p<uint8_t>(),
                                p<int32_t>(), p<int32_t>(), p<int32_t>(), p<int32_t>(),
                                p<int32_t>(), p<int32_t>(), p<float>(), p<int32_t>(), ptr(),
                                pick(kSizes), nullptr);
        break;
      case 3:
        st = ep_regroup_by_expert(ptr(), p<const int32_t>(), p<const float>(), p<const int32_t>(),
                                  pick(kI32), pick(kI64), pick(kI32), pick(kI32), pick(kI32),
                                  pick(kI32), pick(kI64), ptr(), p<int32_t>(), p<float>(),
                                  p<int32_t>(), p<int32_t>(), p<int32_t>(), ptr(), pick(kSizes),
                                  nullptr);
        break;
      case 4:
        st = ep_dispatch_permute(ptr(), pick(kI64), pick(kI32), p<const int32_t>(), pick(kI32),
                                 pick(kI64), int(rng() % 4), ptr(), p<float>(), nullptr);
        break;
      case 5:
        st = ep_batched_prepare(ptr(), p<const int64_t>(), pick(kI64), pick(kI32), pick(kI32),
                                pick(kI32), pick(kI32), pick(kI64), ptr(), p<int32_t>(),
                                p<int32_t>(), ptr(), pick(kSizes), nullptr);
        break;
      case 6:
        st = ep_batched_prepare_fp8(ptr(), p<const int64_t>(), pick(kI64), pick(kI32),
                                    pick(kI32), pick(kI32), pick(kI32), pick(kI64),
                                    int(rng() % 4), int(rng() % 3), ptr(), ptr(), p<int32_t>(),
                                    p<int32_t>(), ptr(), pick(kSizes), nullptr);
        break;
      case 7:
        st = ep_combine(ptr(), pick(kI64), p<const int32_t>(), p<const float>(), pick(kI64),
                        pick(kI32), pick(kI32), ptr(), ptr(), ptr(), nullptr);
        break;
      default: {
        volatile size_t s = ep_counts_workspace_bytes(pick(kI64), pick(kI32), pick(kI32),
                                                      pick(kI32)) +
                            ep_layout_workspace_bytes(pick(kI64), pick(kI32)) +
                            ep_batched_workspace_bytes(pick(kI64), pick(kI32), pick(kI64)) +
                            ep_dispatch_layout_workspace_bytes(pick(kI64), pick(kI32),
                                                               pick(kI32)) +
                            ep_regroup_workspace_bytes(pick(kI64), pick(kI32));
        (void)s;
        (void)ep_status_string(pick(kI32));
        continue;
      }
    }
    if (st == EP_OK || st == EP_ERR_LAUNCH)
      ++passed;
    else if (st == EP_ERR_INVALID_ARG || st == EP_ERR_UNSUPPORTED || st == EP_ERR_WORKSPACE)
      ++rejected;
    else
      return 2;  // not a status the ABI defines
  }
  std::printf("done: %ld rejected, %ld passed validation\n", rejected, passed);
  return 0;
}
