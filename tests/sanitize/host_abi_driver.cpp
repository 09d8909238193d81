// Drives every host-side path of the C ABI that makes no HIP call (size
// queries, argument validation, the codebook, status texts, the timing
// hook) so that an AddressSanitizer / UndefinedBehaviorSanitizer build of
// the library's host code can check them.  Exits 0 when every expected
// status is returned; a sanitizer report ends the process with an error.
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <initializer_list>

#include "qlora_nf4.h"

static int failures = 0;
#define EXPECT(cond)                                                        \
  do {                                                                      \
    if (!(cond)) {                                                          \
      std::fprintf(stderr, "%s:%d: expected %s (%s)\n", __FILE__, __LINE__, \
                   #cond, qlora_last_error());                              \
      ++failures;                                                           \
    }                                                                       \
  } while (0)

int main() {
  void* const F = reinterpret_cast<void*>(uintptr_t(0x7F0000000000ull));  // never dereferenced
  uint8_t* const F8 = static_cast<uint8_t*>(F);
  float* const Ff = static_cast<float*>(F);
  qlora_sizes_t sz;
  // size queries over shapes, ranks and token counts, valid and invalid
  const int64_t shapes[][2] = {{256, 256}, {4096, 4096}, {11008, 4096}, {4096, 11008}, {22016, 8192}, {8, 64}};
  const int32_t ranks[] = {1, 8, 33, 64, 256};
  const int64_t ms[] = {0, 1, 16, 17, 300, 4096, 40000};
  for (auto& s : shapes)
    for (int32_t r : ranks)
      for (int64_t m : ms) {
        EXPECT(qlora_nf4_sizes(s[0], s[1], m, r, &sz) == QLORA_OK);
        EXPECT(sz.codes_bytes == (size_t)(s[0] * s[1] / 2));
      }
  EXPECT(qlora_nf4_sizes(256, 96, 0, 8, &sz) == QLORA_ERR_INVALID_ARG);
  EXPECT(qlora_nf4_sizes(250, 256, 0, 8, &sz) == QLORA_ERR_INVALID_ARG);
  EXPECT(qlora_nf4_sizes(256, 256, -1, 8, &sz) == QLORA_ERR_INVALID_ARG);
  EXPECT(qlora_nf4_sizes(256, 256, 0, 0, &sz) == QLORA_ERR_INVALID_ARG);
  EXPECT(qlora_nf4_sizes(256, 256, 0, 257, &sz) == QLORA_ERR_INVALID_ARG);
  EXPECT(qlora_nf4_sizes(256, 256, 0, 8, nullptr) == QLORA_ERR_INVALID_ARG);
  EXPECT(qlora_nf4_sizes(int64_t(1) << 40, 1 << 20, 0, 8, &sz) == QLORA_ERR_INVALID_ARG);

  qlora_nf4_t w{4096, 4096, F8, F8, Ff, Ff};
  // quantize / dequantize validation
  EXPECT(qlora_nf4_quantize(F, 9, 4096, 4096, &w, F, 1 << 30, nullptr) == QLORA_ERR_UNSUPPORTED_DTYPE);
  EXPECT(qlora_nf4_quantize(F, QLORA_F32, 4096, 4096, &w, F, 16, nullptr) == QLORA_ERR_WORKSPACE_TOO_SMALL);
  EXPECT(qlora_nf4_quantize(nullptr, QLORA_F32, 4096, 4096, &w, F, 1 << 30, nullptr) == QLORA_ERR_INVALID_ARG);
  EXPECT(qlora_dequantize(&w, F, QLORA_F32, nullptr) == QLORA_ERR_UNSUPPORTED_DTYPE);
  EXPECT(qlora_dequantize(nullptr, F, QLORA_BF16, nullptr) == QLORA_ERR_INVALID_ARG);
  // forward / backward: every stop before the launch
  for (int64_t m : {1, 16, 17, 4096}) {
    EXPECT(qlora_linear_fwd(&w, F, m, F, F, 64, 16.f, F, QLORA_BF16, nullptr, F, 0, nullptr) ==
           QLORA_ERR_WORKSPACE_TOO_SMALL || m <= 16);
    EXPECT(qlora_linear_bwd(&w, F, F, m, F, F, 64, 16.f, nullptr, F, QLORA_BF16, Ff, Ff, F, 0, nullptr) ==
           QLORA_ERR_WORKSPACE_TOO_SMALL);
  }
  EXPECT(qlora_linear_fwd(&w, F, -1, F, F, 64, 16.f, F, QLORA_BF16, nullptr, F, 0, nullptr) == QLORA_ERR_INVALID_ARG);
  EXPECT(qlora_linear_fwd(&w, F, 32, F, F, 64, 16.f, F, QLORA_F16, nullptr, F, 0, nullptr) ==
         QLORA_ERR_UNSUPPORTED_DTYPE);
  EXPECT(qlora_linear_fwd_ex(&w, F, 32, F, F, 64, 16.f, F, QLORA_F16, nullptr, F, 0, 7, nullptr) ==
         QLORA_ERR_UNSUPPORTED_DTYPE);
  EXPECT(qlora_linear_bwd_ex(&w, F, F, 32, F, F, 64, 16.f, nullptr, F, QLORA_BF16, Ff, Ff, F, 0, 7, nullptr) ==
         QLORA_ERR_UNSUPPORTED_DTYPE);
  qlora_nf4_t big{22016, 8192, F8, F8, Ff, Ff};
  EXPECT(qlora_linear_fwd(&big, F, 60000, F, F, 64, 16.f, F, QLORA_BF16, nullptr, F, size_t(1) << 40, nullptr) ==
         QLORA_ERR_INVALID_ARG);
  EXPECT(qlora_linear_fwd_noalloc(&big, F, 48000, F, F, 64, 16.f, F, QLORA_BF16, nullptr, nullptr) ==
         QLORA_ERR_WORKSPACE_TOO_SMALL);
  EXPECT(qlora_linear_fwd_noalloc(&w, F, 32, F, F, 0, 16.f, F, QLORA_BF16, nullptr, nullptr) ==
         QLORA_ERR_INVALID_ARG);
  qlora_nf4_t misaligned{4096, 4096, F8 + 4, F8, Ff, Ff};
  EXPECT(qlora_linear_fwd(&misaligned, F, 32, F, F, 8, 16.f, F, QLORA_BF16, nullptr, F, 0, nullptr) ==
         QLORA_ERR_INVALID_ARG);
  // AdamW, merge and the comparison formats
  qlora_adamw_tensor_t t[9];
  std::memset(t, 0, sizeof(t));
  EXPECT(qlora_adamw_step(t, 9, QLORA_BF16, 1e-3f, 0.9f, 0.999f, 1e-8f, 0.f, 1, nullptr) == QLORA_ERR_INVALID_ARG);
  EXPECT(qlora_adamw_step(t, 1, QLORA_BF16, 1e-3f, 1.0f, 0.999f, 1e-8f, 0.f, 1, nullptr) == QLORA_ERR_INVALID_ARG);
  EXPECT(qlora_adamw_step(t, 1, QLORA_BF16, 1e-3f, 0.9f, 0.999f, 1e-8f, 0.f, 0, nullptr) == QLORA_ERR_INVALID_ARG);
  t[0].n = -1;
  EXPECT(qlora_adamw_step(t, 1, QLORA_F32, 1e-3f, 0.9f, 0.999f, 1e-8f, 0.f, 1, nullptr) == QLORA_ERR_INVALID_ARG);
  EXPECT(qlora_merge_lora(&w, F, F, 0, 16.f, F, QLORA_BF16, nullptr) == QLORA_ERR_INVALID_ARG);
  EXPECT(qlora_merge_lora(&w, F, F, 8, 16.f, F, QLORA_F32, nullptr) == QLORA_ERR_UNSUPPORTED_DTYPE);
  qlora_qtensor_t qt{4096, 4096, 9, F8, Ff};
  EXPECT(qlora_quantize_format(F, QLORA_F32, 4096, 4096, &qt, nullptr) == QLORA_ERR_INVALID_ARG);
  qt.format = QLORA_FMT_INT8;
  EXPECT(qlora_dequantize_format(&qt, F, QLORA_F32, nullptr) == QLORA_ERR_UNSUPPORTED_DTYPE);
  EXPECT(qlora_gemv_format(&qt, F, 17, F, QLORA_BF16, nullptr) == QLORA_ERR_INVALID_ARG);
  // helpers
  float cb[16];
  qlora_nf4_codebook(cb);
  EXPECT(cb[0] == -1.0f && cb[7] == 0.0f && cb[15] == 1.0f);
  for (int i = 0; i < 15; ++i) EXPECT(cb[i] < cb[i + 1]);
  qlora_nf4_codebook(nullptr);
  for (int s = -1; s <= 5; ++s) EXPECT(qlora_status_string(s) != nullptr && std::strlen(qlora_status_string(s)) > 0);
  EXPECT(qlora_time_next_launch(99, F, F) == QLORA_ERR_INVALID_ARG);
  EXPECT(qlora_time_next_launch(QLORA_KERNEL_GEMV, nullptr, F) == QLORA_ERR_INVALID_ARG);
  EXPECT(qlora_time_next_launch(QLORA_KERNEL_GEMV, F, F) == QLORA_OK);
  EXPECT(qlora_time_next_launch(QLORA_KERNEL_NONE, nullptr, nullptr) == QLORA_OK);
  if (failures) {
    std::fprintf(stderr, "%d expectation(s) failed\n", failures);
    return 1;
  }
  std::printf("host ABI paths ok\n");
  return 0;
}
