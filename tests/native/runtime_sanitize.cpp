// runtime_sanitize.cpp -- drives the host-only paths of the C ABI
// (quantized_delta_rule_decode_amd/csrc/qdr_runtime.cpp): descriptor checks,
// the pool layout, argument checks of every entry point, qdr_last_error, and
// pool creation on a process that sees no device.  Built with g++ under
// AddressSanitizer / UndefinedBehaviorSanitizer against the HIP runtime's
// host library by tests/test_sanitizers.py; the device launches are replaced
// by the stub below (nothing here may reach a kernel).
//
// Prints "ok <n>" (n = checks passed) and exits 0; a failed check exits 1,
// a sanitizer report aborts.
#include <cmath>
#include <cstdio>
#include <cstring>
#include <vector>

#include "../../include/qdr.h"
#include "../../quantized_delta_rule_decode_amd/csrc/qdr_internal.h"

namespace qdr {
hipError_t launch_all(const PoolConfig &, LaunchArgs, int, const ListEntry *const *, const int32_t *, int,
                      hipStream_t, hipStream_t) {
  std::fprintf(stderr, "a device launch was reached\n");
  std::abort();
}
}  // namespace qdr

static int checks = 0;
#define CHECK(x)                                                      \
  do {                                                                \
    if (!(x)) {                                                       \
      std::fprintf(stderr, "check failed at line %d: %s (%s)\n", __LINE__, #x, qdr_last_error()); \
      return 1;                                                       \
    }                                                                 \
    ++checks;                                                         \
  } while (0)

int main() {
  const int H = 5;
  std::vector<uint8_t> head_kinds = {2, 4, 6, 8, 16};
  std::vector<uint8_t> row_kinds(H * QDR_DIM);
  for (size_t i = 0; i < row_kinds.size(); ++i) row_kinds[i] = (uint8_t)(std::vector<int>{2, 4, 6, 8, 16, 32}[i % 6]);
  std::vector<float> omega(H * QDR_DIM, 1.0f);
  for (int unit = 0; unit < 2; ++unit)
    for (int mode = 0; mode < 2; ++mode)
      for (int sb : {0, 16, 32}) {
        qdr_pool_desc d{};
        d.num_slots = 2561; d.num_heads = H; d.d_k = d.d_v = QDR_DIM;
        d.unit = unit; d.gate = unit; d.scale_mode = mode; d.fit_iters = 0;
        d.kinds = unit ? row_kinds.data() : head_kinds.data();
        d.omega = omega.data(); d.scale_bits = sb;
        size_t n = 0;
        CHECK(qdr_pool_bytes(&d, &n) == QDR_OK && n > 0 && n % 256 == 0);
        CHECK(std::strcmp(qdr_last_error(), "") == 0);
        // invalid descriptors, each rejected with a message
        qdr_pool_desc b = d; b.num_slots = 0;
        CHECK(qdr_pool_bytes(&b, &n) == QDR_E_INVAL && std::strlen(qdr_last_error()) > 0);
        b = d; b.d_k = 64;
        CHECK(qdr_pool_bytes(&b, &n) == QDR_E_UNSUPPORTED);
        b = d; b.fit_iters = 1;
        CHECK(qdr_pool_bytes(&b, &n) == (mode == QDR_SCALE_DUAL ? QDR_OK : QDR_E_INVAL));
        b = d; b.kinds = nullptr;
        CHECK(qdr_pool_bytes(&b, &n) == QDR_E_INVAL);
        std::vector<uint8_t> bad_kinds(unit ? row_kinds : head_kinds);
        bad_kinds.back() = 7;
        b = d; b.kinds = bad_kinds.data();
        CHECK(qdr_pool_bytes(&b, &n) == QDR_E_INVAL);
        std::vector<float> bad_omega(omega);
        bad_omega[3] = std::nanf("");
        b = d; b.omega = bad_omega.data();
        CHECK(qdr_pool_bytes(&b, &n) == (mode == QDR_SCALE_DUAL ? QDR_E_INVAL : QDR_OK));
        CHECK(qdr_pool_bytes(&d, nullptr) == QDR_E_INVAL);
        // creation without a visible device: a device error, nothing returned
        qdr_pool *p = reinterpret_cast<qdr_pool *>(0x1);
        const qdr_status st = qdr_pool_create(&d, nullptr, 0, &p);
        CHECK(st == QDR_E_DEVICE && p == nullptr);
        CHECK(qdr_pool_create(&b, nullptr, 0, &p) != QDR_OK);
      }
  // every entry point rejects a null pool before touching anything
  float f = 0.0f;
  uint32_t flags = 0;
  unsigned char raw[16];
  qdr_layout lay{};
  CHECK(qdr_pool_destroy(nullptr) == QDR_OK);
  CHECK(qdr_slot_reset(nullptr, nullptr, 1, nullptr) == QDR_E_INVAL);
  CHECK(qdr_pack(nullptr, nullptr, 1, &f, nullptr) == QDR_E_INVAL);
  CHECK(qdr_unpack(nullptr, nullptr, 1, &f, nullptr) == QDR_E_INVAL);
  CHECK(qdr_decode_step(nullptr, nullptr, 1, &f, &f, &f, &f, &f, &f, nullptr) == QDR_E_INVAL);
  CHECK(qdr_decode_step_bf16(nullptr, nullptr, 1, nullptr, nullptr, nullptr, &f, &f, nullptr, nullptr) == QDR_E_INVAL);
  CHECK(qdr_decode_step_split(nullptr, nullptr, 1, &f, &f, &f, &f, &f, &f, nullptr, nullptr) == QDR_E_INVAL);
  CHECK(qdr_get_layout(nullptr, &lay) == QDR_E_INVAL);
  CHECK(qdr_read_raw(nullptr, 0, raw, sizeof raw, nullptr) == QDR_E_INVAL);
  CHECK(qdr_write_raw(nullptr, 0, raw, sizeof raw, nullptr) == QDR_E_INVAL);
  CHECK(qdr_poll_device_error(nullptr, &flags) == QDR_E_INVAL);
  CHECK(std::strlen(qdr_last_error()) > 0);
  std::printf("ok %d\n", checks);
  return 0;
}
