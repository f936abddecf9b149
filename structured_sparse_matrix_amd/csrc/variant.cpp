// Environment switches of libsnm, read once per process (host code only):
//   SNM_LOG=1            every product call prints the kernel variant it selects to stderr,
//                        one line: "snm: <operation> R=.. K=.. C=.. -> <variant>".
//   SNM_FORCE_VARIANT=v  prefer variant v where it applies, for A/B comparisons of kernels
//                        on one shape; a variant that does not apply to a call (or an
//                        unknown name) leaves the shape-based choice unchanged:
//                          wide     V:N:M products: the wide-tile kernel, never the large-tile one
//                          large    V:N:M products: the large-tile kernel wherever its shape rules
//                                   hold, whatever the grid size
//                          generic  N:M and canonical V:N:M products: the generic tiled kernel
//                                   (no skinny or wide-tile kernel)
//                          unsplit  split-reduction decode entry points: never split
//                          direct   decode products on operand-major A with column-major B: B
//                                   loaded straight into the operand registers, never
//                                   through the LDS ring
#include "variant.hpp"

#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>

namespace snm {
namespace {

struct Switches {
  bool log = false;
  Variant force = Variant::kNone;
};

const Switches& switches() {
  static Switches s;
  static std::once_flag once;
  std::call_once(once, [] {
    const char* l = std::getenv("SNM_LOG");
    s.log = l != nullptr && l[0] != '\0' && std::strcmp(l, "0") != 0;
    const char* f = std::getenv("SNM_FORCE_VARIANT");
    if (f != nullptr) {
      if (std::strcmp(f, "wide") == 0) s.force = Variant::kWide;
      else if (std::strcmp(f, "large") == 0) s.force = Variant::kLarge;
      else if (std::strcmp(f, "generic") == 0) s.force = Variant::kGeneric;
      else if (std::strcmp(f, "unsplit") == 0) s.force = Variant::kUnsplit;
      else if (std::strcmp(f, "direct") == 0) s.force = Variant::kDirect;
    }
  });
  return s;
}

}  // namespace

Variant forced_variant() { return switches().force; }

void log_variant(const char* op, int64_t R, int64_t K, int64_t C, const char* variant) {
  if (!switches().log) return;
  std::fprintf(stderr, "snm: %s R=%lld K=%lld C=%lld -> %s\n", op, (long long)R, (long long)K,
               (long long)C, variant);
}

}  // namespace snm
