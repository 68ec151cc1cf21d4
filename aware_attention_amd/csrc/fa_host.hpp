// Host helpers shared by the entry points of libfa.so (defined in fa_api.hip).
#pragma once

#include <string>

#include "fa.h"

namespace fa_host {

// Message of the calling thread's most recent failure (fa_last_error).
extern thread_local std::string g_last_error;

// Record msg as the calling thread's last error and return s.
fa_status fail(fa_status s, const std::string& msg);

bool aligned16(const void* ptr);

// FA_OK when the current HIP device is a gfx950 (looked up once per device).
fa_status check_device();

}  // namespace fa_host
