"""MI355X-native shared-routing sparse decode attention (CLSA)."""
