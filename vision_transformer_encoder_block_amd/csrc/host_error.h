// The library's per-thread error message (returned by vit_last_error), shared
// by the encoder and head runtimes.
#pragma once

#include <string>

namespace vit {

// Records `msg` as the calling thread's last error and returns `code`.
int report_error(int code, const std::string& msg);

}  // namespace vit
