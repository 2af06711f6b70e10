// Host-side sweep of every libnvfp4 entry point with invalid, boundary and
// overflowing arguments, for a build whose host code is compiled with
// AddressSanitizer and UndefinedBehaviorSanitizer.  Pointers are fake
// addresses that must never be dereferenced: argument checks run before any
// device work, and on a machine without a GPU every call that passes them
// stops at the device check.  With a GPU present the sweep does not run (a
// call that passed validation would launch on the fake addresses).
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>

#include "nvfp4.h"

namespace {

const int64_t kSizes[] = {-1, 0, 1, 8, 16, 32, 128, 256, 5120, 17408, (int64_t)1 << 31, (int64_t)1 << 40,
                          INT64_MAX / 16, INT64_MAX - 1, INT64_MAX};
const int kNumSizes = sizeof(kSizes) / sizeof(kSizes[0]);

template <typename T>
T* fake(uint64_t base, uint64_t off = 0) {
  return reinterpret_cast<T*>(base + off);
}

const uint64_t A = 0x100000000000ull, B = 0x200000000000ull, C = 0x300000000000ull, D = 0x400000000000ull,
               E = 0x500000000000ull, F = 0x600000000000ull, G = 0x700000000000ull, H = 0x800000000000ull;

long g_calls = 0;
long g_ok = 0;

void note(nvfp4_status st) {
  ++g_calls;
  if (st == NVFP4_OK) ++g_ok;
  if (st < NVFP4_OK || st > NVFP4_ERR_ALIAS) {
    fprintf(stderr, "status out of range: %d\n", (int)st);
    __builtin_trap();
  }
}

}  // namespace

int main() {
  int devices = 0;
  if (hipGetDeviceCount(&devices) == hipSuccess && devices > 0) {
    printf("GPU present: sweep skipped\n");
    return 0;
  }
  for (int s = -3; s < 10; ++s) (void)nvfp4_status_string(s);
  (void)nvfp4_version();
  (void)nvfp4_linear_noalloc_max_bytes();
  (void)nvfp4_quantize_workspace_bytes();
  for (int offs = 0; offs < 3; ++offs) {
    const uint64_t o = offs == 0 ? 0 : (offs == 1 ? 8 : 16);
    for (int i = 0; i < kNumSizes; ++i) {
      const int64_t a = kSizes[i];
      (void)nvfp4_stream_read_sink_words(a);
      note(nvfp4_stream_read(fake<void>(A, o), a, fake<uint32_t>(B), nullptr));
      for (int j = 0; j < kNumSizes; ++j) {
        const int64_t b = kSizes[j];
        (void)nvfp4_prepared_bytes(a, b);
        (void)nvfp4_mx_linear_w4a4_workspace_bytes(a, b);
        (void)nvfp4_linear_w4a4_workspace_bytes(a, b);
        note(nvfp4_quantize(fake<uint16_t>(A, o), a, b, fake<uint8_t>(B), fake<uint8_t>(C), fake<float>(D), nullptr));
        note(nvfp4_amax_accumulate(fake<uint16_t>(A, o), a, b, fake<float>(D), nullptr));
        note(nvfp4_quantize_ws(fake<uint16_t>(A), a, b, fake<uint8_t>(B), fake<uint8_t>(C), fake<float>(D),
                               fake<void>(F, o), a, nullptr));
        note(nvfp4_quantize_with_amax(fake<uint16_t>(A), a, b, fake<float>(D, o), fake<uint8_t>(B), fake<uint8_t>(C),
                                      fake<float>(E), nullptr));
        note(nvfp4_dequant(fake<uint8_t>(B, o), fake<uint8_t>(C), fake<float>(D), a, b, fake<uint16_t>(A), nullptr));
        note(nvfp4_prepare(fake<uint8_t>(B), fake<uint8_t>(C, o), a, b, fake<uint8_t>(E), nullptr));
        note(nvfp4_dequant_prepared(fake<uint8_t>(E, o), fake<float>(D), a, b, fake<uint16_t>(A), nullptr));
        note(nvfp4_mx_quantize(fake<uint16_t>(A, o), a, b, fake<uint8_t>(B), fake<uint8_t>(C), nullptr));
        note(nvfp4_mx_dequant(fake<uint8_t>(B), fake<uint8_t>(C, o), a, b, fake<uint16_t>(A), nullptr));
        for (int l = 0; l < kNumSizes; ++l) {
          const int64_t c = kSizes[l];
          (void)nvfp4_linear_workspace_bytes(a, b, c);
          (void)nvfp4_linear_prepared_workspace_bytes(a, b, c);
          (void)nvfp4_linear_grouped_workspace_bytes(a, b, c);
          note(nvfp4_linear(fake<uint16_t>(A, o), a, b, c, fake<uint8_t>(B), fake<uint8_t>(C), fake<float>(D),
                            fake<uint16_t>(E), nullptr));
          note(nvfp4_linear_ws(fake<uint16_t>(A), a, b, c, fake<uint8_t>(B, o), fake<uint8_t>(C), fake<float>(D),
                               fake<uint16_t>(E), fake<void>(F), c, nullptr));
          note(nvfp4_linear_noalloc(fake<uint16_t>(A), a, b, c, fake<uint8_t>(B), fake<uint8_t>(C), fake<float>(D),
                                    fake<uint16_t>(E, o), nullptr));
          note(nvfp4_linear_prepared(fake<uint16_t>(A), a, b, c, fake<uint8_t>(E, o), fake<float>(D),
                                     fake<uint16_t>(B), fake<void>(F), a, nullptr));
          for (int kid = -1; kid < 5; ++kid)
            note(nvfp4_linear_forced(kid, fake<uint16_t>(A), a, b, c, fake<uint8_t>(B), fake<uint8_t>(C),
                                     fake<float>(D), fake<uint16_t>(E), nullptr));
          note(nvfp4_quantize_experts(fake<uint16_t>(A, o), a, b, c, fake<uint8_t>(B), fake<uint8_t>(C),
                                      fake<float>(D), nullptr));
          note(nvfp4_dequant_experts(fake<uint8_t>(B), fake<uint8_t>(C), fake<float>(D, o), a, b, c,
                                     fake<uint16_t>(A), nullptr));
          note(nvfp4_mx_gemm(fake<uint8_t>(A), fake<uint8_t>(B), a, fake<uint8_t>(C, o), fake<uint8_t>(D), b, c,
                             fake<uint16_t>(E), nullptr));
          note(nvfp4_mx_linear_w4a4(fake<uint16_t>(A), a, b, c, fake<uint8_t>(C), fake<uint8_t>(D, o),
                                    fake<uint16_t>(E), fake<void>(F), b, nullptr));
          note(nvfp4_linear_w4a4(fake<uint16_t>(A), a, b, c, fake<uint8_t>(B), fake<uint8_t>(C), fake<float>(D),
                                 fake<uint16_t>(E, o), fake<void>(F), c, nullptr));
          // Expert routing: (t_count, topk, experts) = (a, b, c), weight 256 x 512.
          note(nvfp4_linear_routed(fake<uint16_t>(A), a, b, fake<int32_t>(G, o), c, 256, 512, fake<uint8_t>(B),
                                   fake<uint8_t>(C), fake<float>(D), fake<uint16_t>(E), nullptr));
          note(nvfp4_linear_grouped(fake<uint16_t>(A), a, b, fake<int32_t>(G), c, 256, 512, fake<uint8_t>(B, o),
                                    fake<uint8_t>(C), fake<float>(D), fake<uint16_t>(E), fake<void>(F), a, nullptr));
          // Paged KV gather: (num_blocks, block_size, heads) = (a, b, c), head_dim 128, 4 sequences.
          for (int fmt = 0; fmt < 3; ++fmt)
            note(nvfp4_kv_gather(fmt, fmt & 1, fake<uint8_t>(A), fake<uint8_t>(B), fake<float>(C), a, b, c, 128,
                                 fake<int32_t>(D, o), 16, fake<int32_t>(E), fake<int32_t>(F), 4, fake<uint16_t>(H),
                                 a, nullptr));
        }
      }
    }
  }
  printf("%ld calls, %ld returned OK (no-op shapes)\n", g_calls, g_ok);
  return 0;
}
