// libtaco kernels for E4M3 codes (one translation unit per code format keeps
// each compilation small; see taco_kernels.hpp for the kernels).
#include "taco_kernels.hpp"

template struct taco_internal::Ops<taco_internal::Fmt::kE4M3>;
